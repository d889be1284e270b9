// K2: split-K flash decode over the R-SWA key set (prefix u window), and its cross-split merge.
//
// For sequence b and head h the live keys are the contiguous cache rows [0, L_b), with
// L_b = m_b + min(n_b, t_b) in R-SWA mode (the static prefix then the ring slots in use) or
// m_b + t_b in full-causal mode; the ring's slot order is irrelevant because softmax attention is
// invariant under key permutation. (Key set: deep dive "Unlimited-OCR", N(t) code block; cache
// size: GeekNews "Unlimited OCR", KV cache management section.)
//
// Work decomposition. Each (b, h) key range is cut into chunks of `chunk` rows; an item is one
// (b, h, chunk). A fixed grid of persistent 256-thread workgroups walks the item list, which every
// workgroup derives on the device from the step counters (so no host sync and no per-step table
// upload), with chunk counts a smooth function of L_b.
//
// Inside an item. A row of K or V is 256 B (bf16) or 512 B (fp32): 16 or 32 lanes each load 16 B
// of it, so a wave streams 4 (bf16) or 2 (fp32) rows per load instruction, 1 KiB contiguous.
// Each lane group keeps its own float32 online-softmax state (running max in the log2 domain,
// running sum, and its 8 or 4 output dims); q.k partial dots are summed across the group with DPP
// row operations. At the end of the item the 16 (or 8) group states are merged through LDS; a
// single-chunk (b, h) writes its output directly, otherwise the item leaves a partial
// (max, sum, numerator[128]) in the workspace and a second kernel merges the partials:
//   o = sum_s 2^(M_s - M) A_s / sum_s 2^(M_s - M) l_s,   M = max_s M_s.
// All arithmetic after the bf16 loads is float32.
#include "device.h"
#include "kernels.h"

namespace rswa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxGroups = kWaves * 4;  // bf16: 4 row groups per wave

template <typename KV> struct Lanes;
template <> struct Lanes<uint16_t> { static constexpr int VEC = 8, GL = 16; };
template <> struct Lanes<float> { static constexpr int VEC = 4, GL = 32; };

__device__ __forceinline__ int live_rows(const DecodeArgs& a, int b) {
  if (a.active && !a.active[b]) return 0;
  return a.meta.prefix_len[b] + min(a.meta.steps[b], a.meta.cap[b]);
}

// s_cum[0..B] = exclusive prefix sums of items per sequence, s_len[b] = live rows of b.
__device__ void build_work_table(const DecodeArgs& a, int* s_cum, int* s_len) {
  __shared__ int s_wave_tot[kWaves];
  __shared__ int s_carry;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  if (tid == 0) {
    s_carry = 0;
    s_cum[0] = 0;
  }
  for (int base = 0; base < a.batch; base += kThreads) {
    const int b = base + tid;
    int items = 0;
    if (b < a.batch) {
      const int L = live_rows(a, b);
      s_len[b] = L;
      items = a.heads * ((L + a.chunk - 1) / a.chunk);
    }
    int x = items;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == kWave - 1) s_wave_tot[wave] = x;
    __syncthreads();
    int prefix = s_carry;
    for (int w = 0; w < wave; ++w) prefix += s_wave_tot[w];
    if (b < a.batch) s_cum[b + 1] = prefix + x;
    __syncthreads();
    if (tid == kThreads - 1) s_carry = prefix + x;
  }
  __syncthreads();
}

template <typename KV>
__device__ __forceinline__ float partial_dot(const uint4& q, const uint4& k);

template <>
__device__ __forceinline__ float partial_dot<uint16_t>(const uint4& q, const uint4& k) {
  float s = 0.f;
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.x),
                                      __builtin_bit_cast(bf16x2_t, k.x), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.y),
                                      __builtin_bit_cast(bf16x2_t, k.y), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.z),
                                      __builtin_bit_cast(bf16x2_t, k.z), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w),
                                      __builtin_bit_cast(bf16x2_t, k.w), s, false);
  return s;
}

template <>
__device__ __forceinline__ float partial_dot<float>(const uint4& q, const uint4& k) {
  float s = __uint_as_float(q.x) * __uint_as_float(k.x);
  s = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), s);
  s = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), s);
  s = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), s);
  return s;
}

template <typename KV>
__device__ __forceinline__ float group_sum(float x);
template <>
__device__ __forceinline__ float group_sum<uint16_t>(float x) { return row16_sum(x); }
template <>
__device__ __forceinline__ float group_sum<float>(float x) { return lane32_sum(x); }

template <typename KV>
__device__ __forceinline__ void unpack_v(const uint4& v, float* f);
template <>
__device__ __forceinline__ void unpack_v<uint16_t>(const uint4& v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}
template <>
__device__ __forceinline__ void unpack_v<float>(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

template <typename KV, typename OUT, int U>
__device__ __forceinline__ void decode_item(const DecodeArgs& a, int b, int h, int c, int L,
                                            int nch, float* s_m, float* s_l, float* s_acc) {
  constexpr int VEC = Lanes<KV>::VEC, GL = Lanes<KV>::GL, G = kWave / GL, NG = kWaves * G;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int g = lane / GL, li = lane % GL;
  const int H = a.heads;
  const int64_t R = a.meta.rows[b];
  const KV* seq = reinterpret_cast<const KV*>(a.storage) + a.meta.seq_off[b];
  const KV* Kp = seq + (int64_t)h * R * kHeadDim + li * VEC;
  const KV* Vp = seq + (int64_t)(H + h) * R * kHeadDim + li * VEC;
  const int r0 = c * a.chunk;
  const int r1 = min(r0 + a.chunk, L);
  const uint4 qv = *reinterpret_cast<const uint4*>(reinterpret_cast<const KV*>(a.q) +
                                                   ((int64_t)b * H + h) * kHeadDim + li * VEC);
  float m_run = kNegBig, l_run = 0.f;
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;

  for (int rb = r0 + wave * (G * U); rb < r1; rb += kWaves * G * U) {
    uint4 kr[U], vr[U];
    int row[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      row[u] = rb + u * G + g;
      const int rr = min(row[u], r1 - 1);
      kr[u] = *reinterpret_cast<const uint4*>(Kp + (int64_t)rr * kHeadDim);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rr = min(row[u], r1 - 1);
      vr[u] = *reinterpret_cast<const uint4*>(Vp + (int64_t)rr * kHeadDim);
    }
    float s[U];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float d = group_sum<KV>(partial_dot<KV>(qv, kr[u]));
      s[u] = row[u] < r1 ? d * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[u]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = fast_exp2(s[u] - m_new);
      l_run += p;
      float vf[VEC];
      unpack_v<KV>(vr[u], vf);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = fmaf(p, vf[i], acc[i]);
    }
    m_run = m_new;
  }

  const int gid = wave * G + g;
#pragma unroll
  for (int i = 0; i < VEC; ++i) s_acc[gid * kHeadDim + li * VEC + i] = acc[i];
  if (li == 0) {
    s_m[gid] = m_run;
    s_l[gid] = l_run;
  }
  __syncthreads();
  if (tid < kHeadDim) {
    float M = kNegBig;
#pragma unroll
    for (int k = 0; k < NG; ++k) M = fmaxf(M, s_m[k]);
    float lsum = 0.f, num = 0.f;
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const float w = fast_exp2(s_m[k] - M);
      lsum = fmaf(s_l[k], w, lsum);
      num = fmaf(s_acc[k * kHeadDim + tid], w, num);
    }
    const int64_t bh = (int64_t)b * H + h;
    if (nch == 1) {
      store_out(reinterpret_cast<OUT*>(a.out) + bh * kHeadDim + tid, num / lsum);
    } else {
      const int64_t slot = bh * a.smax + c;
      a.ws_acc[slot * kHeadDim + tid] = num;
      if (tid == 0) a.ws_ml[slot] = make_float2(M, lsum);
    }
  }
  __syncthreads();
}

template <typename KV, typename OUT, int U>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  extern __shared__ int s_dyn[];
  __shared__ float s_m[kMaxGroups], s_l[kMaxGroups];
  __shared__ float s_acc[kMaxGroups * kHeadDim];
  int* s_cum = s_dyn;
  int* s_len = s_dyn + a.batch + 1;
  build_work_table(a, s_cum, s_len);
  const int total = s_cum[a.batch];
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    int lo = 0, hi = a.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_cum[mid] <= w) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int L = s_len[b];
    const int nch = (L + a.chunk - 1) / a.chunk;
    const int local = w - s_cum[b];
    const int h = local / nch;
    const int c = local - h * nch;
    decode_item<KV, OUT, U>(a, b, h, c, L, nch, s_m, s_l, s_acc);
  }
}

template <typename OUT>
__global__ __launch_bounds__(kHeadDim) void decode_merge_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.heads;
  const int L = live_rows(a, b);
  const int nch = (L + a.chunk - 1) / a.chunk;
  if (nch <= 1) return;  // inactive (L = 0) or written directly by decode_kernel
  const int tid = threadIdx.x;
  const int64_t slot0 = (int64_t)bh * a.smax;
  float M = kNegBig;
  for (int s = 0; s < nch; ++s) M = fmaxf(M, a.ws_ml[slot0 + s].x);
  float lsum = 0.f, num = 0.f;
  for (int s = 0; s < nch; ++s) {
    const float2 ml = a.ws_ml[slot0 + s];
    const float w = fast_exp2(ml.x - M);
    lsum = fmaf(ml.y, w, lsum);
    num = fmaf(a.ws_acc[(slot0 + s) * kHeadDim + tid], w, num);
  }
  store_out(reinterpret_cast<OUT*>(a.out) + (int64_t)bh * kHeadDim + tid, num / lsum);
}

template <typename KV, typename OUT>
hipError_t launch_typed(const DecodeArgs& a, int grid, bool need_merge, hipStream_t s) {
  const size_t smem = (size_t)(2 * a.batch + 1) * sizeof(int);
  if (grid > 0) {
    hipLaunchKernelGGL((decode_kernel<KV, OUT, 4>), dim3(grid), dim3(kThreads), smem, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (need_merge) {
    hipLaunchKernelGGL((decode_merge_kernel<OUT>), dim3(a.batch * a.heads), dim3(kHeadDim), 0, s,
                       a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int kv_f32, int out_f32, int grid_blocks,
                         bool need_merge, hipStream_t s) {
  if (kv_f32) {
    return out_f32 ? launch_typed<float, float>(a, grid_blocks, need_merge, s)
                   : launch_typed<float, uint16_t>(a, grid_blocks, need_merge, s);
  }
  return out_f32 ? launch_typed<uint16_t, float>(a, grid_blocks, need_merge, s)
                 : launch_typed<uint16_t, uint16_t>(a, grid_blocks, need_merge, s);
}

}  // namespace rswa
