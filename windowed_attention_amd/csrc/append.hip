// K1: ring append / evict, and the one-time prefix copy of cache creation.
//
// The pages hold the decode cache as a queue of capacity m + n from which every new token evicts
// the oldest output KV (deep dive "Unlimited-OCR", N(t) code block; GeekNews "Unlimited OCR",
// model architecture section). Here the queue's output part is an n-slot ring: output index j
// (0-based) is written to row m + (j mod n), overwriting output j - n, so an append is one row
// write per head with no data movement, and the live rows are always the contiguous range
// [0, m + min(n, t)). Full-causal mode writes row m + j (the cache grows, standard attention).
// The prefix rows [0, m) are written once at creation and never again (GeekNews, DeepEncoder
// section: visual tokens are encoded once and stay static); a paged prefix is not in the cache
// at all, and the output rows then start at storage row 0.
#include "device.h"
#include "kernels.h"

namespace rswa {
namespace {

constexpr int kThreads = 256;

// One workgroup per sequence. Counters are double-buffered: t_b is read from steps_in and
// t_b + (appended) written to steps_out, so no workgroup of this launch races on them.
template <int ELEM>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  const int t = a.steps_in[b];
  if (a.active && !a.active[b]) {
    if (threadIdx.x == 0) a.steps_out[b] = t;
    return;
  }
  const int cap = a.meta.cap[b];
  if (a.full_causal && t >= cap) {
    if (threadIdx.x == 0) {
      *a.meta.err = 1;
      a.steps_out[b] = t;
    }
    return;
  }
  // storage row of the new output: after the prefix, or from row 0 when the prefix is paged
  const int64_t m0 = a.meta.table ? 0 : a.meta.prefix_len[b];
  const int64_t row = a.full_causal ? m0 + t : m0 + t % cap;
  const int64_t R = a.meta.rows[b];
  constexpr int CH = kHeadDim * ELEM / 16;  // 16-byte pieces per row
  const int H = a.heads;
  char* seq = reinterpret_cast<char*>(a.storage) + a.meta.seq_off[b] * ELEM;
  const char* kin = reinterpret_cast<const char*>(a.k_new);
  const char* vin = reinterpret_cast<const char*>(a.v_new);
  for (int i = threadIdx.x; i < H * CH; i += kThreads) {
    const int h = i / CH, c = i - (i / CH) * CH;
    const int64_t src = ((int64_t)b * H + h) * kHeadDim * ELEM + c * 16;
    const int64_t dk = ((int64_t)h * R + row) * kHeadDim * ELEM + c * 16;
    const int64_t dv = ((int64_t)(H + h) * R + row) * kHeadDim * ELEM + c * 16;
    const uint4 kx = *reinterpret_cast<const uint4*>(kin + src);
    const uint4 vx = *reinterpret_cast<const uint4*>(vin + src);
    *reinterpret_cast<uint4*>(seq + dk) = kx;
    *reinterpret_cast<uint4*>(seq + dv) = vx;
  }
  if (threadIdx.x == 0) a.steps_out[b] = t + 1;
}

// Packed token-major prefix [sum m][H][D] -> head-major rows [0, m_b) of sequence b.
template <int ELEM>
__global__ __launch_bounds__(kThreads) void prefix_copy_kernel(PrefixCopyArgs a) {
  const int b = blockIdx.y;
  const int64_t m = a.meta.prefix_len[b];
  const int64_t R = a.meta.rows[b];
  constexpr int CH = kHeadDim * ELEM / 16;
  const int H = a.heads;
  const int64_t total = m * H * CH;
  const int64_t row0 = a.prefix_row0[b];
  char* seq = reinterpret_cast<char*>(a.storage) + a.meta.seq_off[b] * ELEM;
  const char* pk = reinterpret_cast<const char*>(a.pk);
  const char* pv = reinterpret_cast<const char*>(a.pv);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t r = i / (H * CH);
    const int rem = (int)(i - r * (H * CH));
    const int h = rem / CH, c = rem - (rem / CH) * CH;
    const int64_t src = ((row0 + r) * H + h) * kHeadDim * ELEM + c * 16;
    const int64_t dk = ((int64_t)h * R + r) * kHeadDim * ELEM + c * 16;
    const int64_t dv = ((int64_t)(H + h) * R + r) * kHeadDim * ELEM + c * 16;
    *reinterpret_cast<uint4*>(seq + dk) = *reinterpret_cast<const uint4*>(pk + src);
    *reinterpret_cast<uint4*>(seq + dv) = *reinterpret_cast<const uint4*>(pv + src);
  }
}

// The live output rows of a cache filled from a packed prefill batch, written as the appends of
// the sequence's t outputs would have left them: in R-SWA mode ring slot q (storage row m + q,
// q < min(n, t)) holds the latest output j < t with j mod n = q, j = t - 1 - ((t - 1 - q) mod n);
// in full-causal mode row m + j holds output j.
template <int ELEM>
__global__ __launch_bounds__(kThreads) void fill_outputs_kernel(FillArgs a) {
  const int b = blockIdx.y;
  const int64_t m = a.meta.prefix_len[b];
  const int t = a.steps[b];
  const int n = a.meta.cap[b];
  const int live = a.full_causal ? t : min(t, n);
  const int64_t R = a.meta.rows[b];
  constexpr int CH = kHeadDim * ELEM / 16;
  const int H = a.heads;
  const int64_t total = (int64_t)live * H * CH;
  const int64_t out0 = a.row0[b] + m;  // packed row of output 0
  char* seq = reinterpret_cast<char*>(a.storage) + a.meta.seq_off[b] * ELEM;
  const char* pk = reinterpret_cast<const char*>(a.k);
  const char* pv = reinterpret_cast<const char*>(a.v);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int q = (int)(i / (H * CH));
    const int rem = (int)(i - (int64_t)q * (H * CH));
    const int h = rem / CH, c = rem - (rem / CH) * CH;
    const int j = a.full_causal ? q : t - 1 - (t - 1 - q) % n;
    const int64_t src = ((out0 + j) * H + h) * kHeadDim * ELEM + c * 16;
    const int64_t r = m + q;
    const int64_t dk = ((int64_t)h * R + r) * kHeadDim * ELEM + c * 16;
    const int64_t dv = ((int64_t)(H + h) * R + r) * kHeadDim * ELEM + c * 16;
    *reinterpret_cast<uint4*>(seq + dk) = *reinterpret_cast<const uint4*>(pk + src);
    *reinterpret_cast<uint4*>(seq + dv) = *reinterpret_cast<const uint4*>(pv + src);
  }
}

__global__ __launch_bounds__(kThreads) void table_check_kernel(const int32_t* table, int64_t n,
                                                               int64_t pool_rows, int32_t* bad) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    const int32_t r = table[i];
    if (r < 0 || r >= pool_rows) *bad = 1;
  }
}

}  // namespace

hipError_t launch_table_check(const int32_t* table, int64_t n, int64_t pool_rows, int32_t* bad,
                              hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t gx = (n + kThreads - 1) / kThreads;
  if (gx > 4096) gx = 4096;
  hipLaunchKernelGGL(table_check_kernel, dim3((unsigned)gx), dim3(kThreads), 0, s, table, n,
                     pool_rows, bad);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, int batch, int kv_f32, hipStream_t s) {
  if (kv_f32)
    hipLaunchKernelGGL(append_kernel<4>, dim3(batch), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(append_kernel<2>, dim3(batch), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefix_copy(const PrefixCopyArgs& a, int kv_f32, int max_rows, hipStream_t s) {
  if (max_rows <= 0) return hipSuccess;
  const int elem = kv_f32 ? 4 : 2;
  const int64_t pieces = (int64_t)max_rows * a.heads * (kHeadDim * elem / 16);
  int64_t gx = (pieces + kThreads - 1) / kThreads;
  if (gx > 4096) gx = 4096;
  if (kv_f32)
    hipLaunchKernelGGL(prefix_copy_kernel<4>, dim3((unsigned)gx, a.batch), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(prefix_copy_kernel<2>, dim3((unsigned)gx, a.batch), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fill_outputs(const FillArgs& a, int kv_f32, int max_rows, hipStream_t s) {
  if (max_rows <= 0) return hipSuccess;
  const int elem = kv_f32 ? 4 : 2;
  const int64_t pieces = (int64_t)max_rows * a.heads * (kHeadDim * elem / 16);
  int64_t gx = (pieces + kThreads - 1) / kThreads;
  if (gx > 4096) gx = 4096;
  if (kv_f32)
    hipLaunchKernelGGL(fill_outputs_kernel<4>, dim3((unsigned)gx, a.batch), dim3(kThreads), 0, s,
                       a);
  else
    hipLaunchKernelGGL(fill_outputs_kernel<2>, dim3((unsigned)gx, a.batch), dim3(kThreads), 0, s,
                       a);
  return hipGetLastError();
}

}  // namespace rswa
