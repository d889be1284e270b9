// K2: flash decode over the R-SWA key set (prefix u window), optionally fused with K1's append,
// and the merge of split partial results.
//
// For sequence b and head h the live keys are the contiguous cache rows [0, L_b), with
// L_b = m_b + min(n_b, t_b) in R-SWA mode (the static prefix then the ring slots in use) or
// m_b + t_b in full-causal mode; the ring's slot order is irrelevant because softmax attention is
// invariant under key permutation. (Key set: deep dive "Unlimited-OCR", N(t) code block; cache
// size: GeekNews "Unlimited OCR", KV cache management section.)
//
// Work decomposition. Every workgroup derives the plan on the device from the step counters, so a
// step needs no host sync and no table upload:
//  * aligned: one 256-thread workgroup per (b, h) key range, used when the batch's ranges are
//    equal and about fill one round of resident workgroups;
//  * stream-K: the concatenation of all (b, h) key ranges is cut into equal contiguous pieces, one
//    per resident workgroup, so every workgroup streams the same number of rows (no tail round,
//    balanced for ragged batches). A piece may cover parts of several ranges; a range split over
//    several pieces leaves float32 partials (max, sum, numerator[128]) that a second kernel merges:
//      o = sum_s 2^(M_s - M) A_s / sum_s 2^(M_s - M) l_s,   M = max_s M_s.
//
// Inside a piece. A row of K or V is 256 B (bf16) or 512 B (fp32): 16 or 32 lanes each load 16 B of
// it, so a wave streams 4 (bf16) or 2 (fp32) rows per load instruction, 1 KiB contiguous. Load
// latency is covered by the other resident waves of the CU (loading the next tile into registers
// ahead of the current one's reduction, RSWA_DECODE_PREFETCH=1, measured no faster and costs
// registers, so it is off). Each lane group keeps its own
// float32 online-softmax state (running max in the log2 domain, running sum, 8 or 4 output dims);
// q.k partial dot products are summed across the group with DPP row operations. At the end of a
// range the group states are merged through LDS.
//
// Fused append (K1 inside K2). When the launch carries the new k/v rows, the new row's slot
// r = m_b + (t_b mod n_b) (or m_b + t_b) is part of the live range after the append; the lane group
// that meets this row in its piece takes k/v from the input instead of the cache and writes them
// into the slot, so no other workgroup reads the slot during the launch and the evicted output is
// never seen.
#include "device.h"
#include "kernels.h"

namespace rswa {
namespace {

#ifndef RSWA_DECODE_PREFETCH
#define RSWA_DECODE_PREFETCH 0  // 1: load the next row tile while reducing the current one
#endif

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxGroups = kWaves * 4;  // bf16: 4 row groups per wave

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename KV> struct Lanes;
template <> struct Lanes<uint16_t> { static constexpr int VEC = 8, GL = 16; };
template <> struct Lanes<float> { static constexpr int VEC = 4, GL = 32; };

// Live rows of sequence b after this launch's append (0 if inactive), and whether it appends.
struct SeqState {
  int L;
  int t;       // step counter before the launch
  bool app;    // this launch appends for b
};

__device__ __forceinline__ SeqState seq_state(const DecodeArgs& a, int b) {
  SeqState st;
  const bool act = !a.active || a.active[b];
  st.t = a.steps_in[b];
  const int cap = a.meta.cap[b];
  st.app = act && a.k_new != nullptr && (!a.full_causal || st.t < cap);
  const int t_after = st.app ? st.t + 1 : st.t;
  st.L = act ? a.meta.prefix_len[b] + min(t_after, cap) : 0;
  return st;
}

// Work table in LDS: s_len[b] = live rows, s_new[b] = cache row of this launch's new k/v (or -1),
// s_cum[b] = sum over b' < b of H * L_b' (int64). Block 0 also publishes the plan for the merge
// kernel and advances the step counters.
__device__ void build_work_table(const DecodeArgs& a, int* s_len, int* s_new, int64_t* s_cum) {
  __shared__ int64_t s_wave_tot[kWaves];
  __shared__ int64_t s_carry;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  if (tid == 0) {
    s_carry = 0;
    s_cum[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < a.batch; base += kThreads) {
    const int b = base + tid;
    int64_t rows = 0;
    if (b < a.batch) {
      const SeqState st = seq_state(a, b);
      s_len[b] = st.L;
      rows = (int64_t)a.heads * st.L;
      int rnew = -1;
      const int m = a.meta.prefix_len[b];
      if (st.app) rnew = a.full_causal ? m + st.t : m + st.t % a.meta.cap[b];
      s_new[b] = rnew;
      if (blockIdx.x == 0) {
        if (a.steps_out) a.steps_out[b] = st.app ? st.t + 1 : st.t;
        if (a.k_new && a.full_causal && (!a.active || a.active[b]) && st.t >= a.meta.cap[b])
          *a.meta.err = 1;
      }
    }
    int64_t x = rows;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int64_t y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == kWave - 1) s_wave_tot[wave] = x;
    __syncthreads();
    int64_t prefix = s_carry;
    for (int w = 0; w < wave; ++w) prefix += s_wave_tot[w];
    if (b < a.batch) s_cum[b + 1] = prefix + x;
    __syncthreads();
    if (tid == kThreads - 1) s_carry = prefix + x;
  }
  __syncthreads();
}

__device__ __forceinline__ int64_t piece_rows(const DecodeArgs& a, int64_t total) {
  const int64_t g = gridDim.x;
  return max((int64_t)a.min_rows, (total + g - 1) / g);
}

template <typename KV>
__device__ __forceinline__ float partial_dot(const u32x4& q, const u32x4& k);

template <>
__device__ __forceinline__ float partial_dot<uint16_t>(const u32x4& q, const u32x4& k) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // copy each element out first: a bit_cast of the element lvalue q[i] reads element 0
    const uint32_t qi = q[i], ki = k[i];
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qi),
                                        __builtin_bit_cast(bf16x2_t, ki), s, false);
  }
  return s;
}

template <>
__device__ __forceinline__ float partial_dot<float>(const u32x4& q, const u32x4& k) {
  float s = __uint_as_float(q[0]) * __uint_as_float(k[0]);
#pragma unroll
  for (int i = 1; i < 4; ++i) s = fmaf(__uint_as_float(q[i]), __uint_as_float(k[i]), s);
  return s;
}

template <typename KV>
__device__ __forceinline__ float group_sum(float x);
template <>
__device__ __forceinline__ float group_sum<uint16_t>(float x) { return row16_sum(x); }
template <>
__device__ __forceinline__ float group_sum<float>(float x) { return lane32_sum(x); }

template <typename KV>
__device__ __forceinline__ void unpack_v(const u32x4& v, float* f);
template <>
__device__ __forceinline__ void unpack_v<uint16_t>(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(v[i]);
    f[2 * i + 1] = bf16_hi(v[i]);
  }
}
template <>
__device__ __forceinline__ void unpack_v<float>(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Combine the np partials of range s stored at workspace slots f + s .. f + s + np - 1 and write
// the output; threads [0, 128) hold one output dim each. (Merging inside the decode kernel, by the
// last workgroup to publish a partial, needs agent-scope release/acquire fences in every
// workgroup; measured on MI355X that costs about 5x the whole step, so the merge is its own
// launch.)
// The (max, sum) pairs are loaded in parallel and reduced in LDS; the numerators are accumulated
// with independent loads, so the merge costs a few memory round trips, not one per partial.
constexpr int kMergeChunk = kHeadDim;
constexpr int kMergeFast = 16;  // pieces per range merged from registers in one memory round trip

template <typename OUT>
__device__ __forceinline__ void merge_range(const DecodeArgs& a, int64_t s, int64_t f, int np,
                                            float* s_w, float* s_l, float* s_red) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  constexpr int NW = kHeadDim / kWave;
  const bool worker = tid < kHeadDim;
  const float2* ml = a.ws_ml + f + s;
  const float* acc = a.ws_acc + (f + s) * kHeadDim + (worker ? tid : 0);
  float M = kNegBig;
  if (np <= kMergeFast) {
    // Few pieces (the usual case): every partial of the range is requested at once, so the merge
    // waits for memory once instead of once per dependent step.
    const float2 p = tid < np ? ml[tid] : make_float2(kNegBig, 0.f);
    float x[kMergeFast];
#pragma unroll
    for (int i = 0; i < kMergeFast; ++i) x[i] = i < np ? acc[(int64_t)i * kHeadDim] : 0.f;
    M = p.x;
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    if (lane == 0 && wave < NW) s_red[wave] = M;
    __syncthreads();
    M = s_red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_red[w]);
    if (tid < np) {
      s_w[tid] = fast_exp2(p.x - M);
      s_l[tid] = p.y;
    }
    __syncthreads();
    float lsum = 0.f, num = 0.f;
#pragma unroll
    for (int i = 0; i < kMergeFast; ++i)
      if (i < np) {
        num = fmaf(x[i], s_w[i], num);
        lsum = fmaf(s_l[i], s_w[i], lsum);
      }
    if (worker) store_out(reinterpret_cast<OUT*>(a.out) + s * kHeadDim + tid, num / lsum);
    __syncthreads();
    return;
  }
  if (worker)
    for (int i = tid; i < np; i += kHeadDim) M = fmaxf(M, ml[i].x);
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0 && wave < NW) s_red[wave] = M;
  __syncthreads();
  M = s_red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, s_red[w]);
  float lsum = 0.f, num = 0.f;
  for (int c = 0; c < np; c += kMergeChunk) {
    const int n = min(kMergeChunk, np - c);
    __syncthreads();
    if (tid < n) {
      const float2 p = ml[c + tid];
      s_w[tid] = fast_exp2(p.x - M);
      s_l[tid] = p.y;
    }
    __syncthreads();
    if (worker) {
      int i = 0;
      for (; i + 4 <= n; i += 4) {
        const float x0 = acc[(int64_t)(c + i) * kHeadDim];
        const float x1 = acc[(int64_t)(c + i + 1) * kHeadDim];
        const float x2 = acc[(int64_t)(c + i + 2) * kHeadDim];
        const float x3 = acc[(int64_t)(c + i + 3) * kHeadDim];
        num = fmaf(x0, s_w[i], num);
        num = fmaf(x1, s_w[i + 1], num);
        num = fmaf(x2, s_w[i + 2], num);
        num = fmaf(x3, s_w[i + 3], num);
      }
      for (; i < n; ++i) num = fmaf(acc[(int64_t)(c + i) * kHeadDim], s_w[i], num);
      for (int j = 0; j < n; ++j) lsum = fmaf(s_l[j], s_w[j], lsum);
    }
  }
  if (worker) store_out(reinterpret_cast<OUT*>(a.out) + s * kHeadDim + tid, num / lsum);
  __syncthreads();
}

// Stream rows [r0, r1) of range (b, h); finish with the group merge through LDS, then either the
// output (the range is not split) or a partial in workspace slot `slot`.
template <typename KV, typename OUT, int U>
__device__ __forceinline__ void decode_range(const DecodeArgs& a, int b, int h, int r0, int r1,
                                             int rnew, bool direct, int64_t slot, float* s_m,
                                             float* s_l, float* s_acc) {
  constexpr int VEC = Lanes<KV>::VEC, GL = Lanes<KV>::GL, G = kWave / GL, NG = kWaves * G;
  constexpr int STEP = kWaves * G * U;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int g = lane / GL, li = lane % GL;
  const int H = a.heads;
  const int64_t R = a.meta.rows[b];
  const int m = a.meta.prefix_len[b];
  // Cache row r lives at Kp + r * D; with a paged prefix the storage starts at row m, and rows
  // r < m are pool rows found through the page table (one 4-byte lookup per row and group).
  const bool paged = a.meta.table != nullptr;
  const int64_t shift = paged ? m : 0;
  KV* seq = reinterpret_cast<KV*>(a.storage) + a.meta.seq_off[b];
  KV* Kp = seq + ((int64_t)h * R - shift) * kHeadDim + li * VEC;
  KV* Vp = seq + ((int64_t)(H + h) * R - shift) * kHeadDim + li * VEC;
  const int32_t* tab = paged ? a.meta.table + a.meta.table_off[b] : nullptr;
  const KV* PKp = paged ? reinterpret_cast<const KV*>(a.meta.pool_k) + h * kHeadDim + li * VEC
                        : nullptr;
  const KV* PVp = paged ? reinterpret_cast<const KV*>(a.meta.pool_v) + h * kHeadDim + li * VEC
                        : nullptr;
  const int64_t pool_stride = (int64_t)H * kHeadDim;
  const int64_t bh = (int64_t)b * H + h;
  const u32x4 qv = ld16(reinterpret_cast<const KV*>(a.q) + bh * kHeadDim + li * VEC);
  const KV* kin = a.k_new ? reinterpret_cast<const KV*>(a.k_new) + bh * kHeadDim + li * VEC : nullptr;
  const KV* vin = a.v_new ? reinterpret_cast<const KV*>(a.v_new) + bh * kHeadDim + li * VEC : nullptr;

  float m_run = kNegBig, l_run = 0.f;
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;

  u32x4 kc[U], vc[U];
  int rb = r0 + wave * (G * U);
  auto load = [&](int base, u32x4* kr, u32x4* vr) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = base + u * G + g;
      const int rr = min(row, r1 - 1);
      const bool fresh = rr == rnew;
      if (paged && rr < m) {
        const int64_t pr = (int64_t)tab[rr] * pool_stride;
        kr[u] = ld16(PKp + pr);
        vr[u] = ld16(PVp + pr);
      } else {
        kr[u] = ld16(fresh ? kin : Kp + (int64_t)rr * kHeadDim);
        vr[u] = ld16(fresh ? vin : Vp + (int64_t)rr * kHeadDim);
      }
    }
  };
  if (rb < r1) load(rb, kc, vc);
  for (; rb < r1; rb += STEP) {
    u32x4 kn[U], vn[U];
    const bool more = rb + STEP < r1;
    if (RSWA_DECODE_PREFETCH && more) load(rb + STEP, kn, vn);
    float s[U];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = rb + u * G + g;
      const float d = group_sum<KV>(partial_dot<KV>(qv, kc[u]));
      s[u] = row < r1 ? d * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[u]);
      if (row == rnew && row < r1) {  // the new row: store it into its slot
        *reinterpret_cast<u32x4*>(Kp + (int64_t)row * kHeadDim) = kc[u];
        *reinterpret_cast<u32x4*>(Vp + (int64_t)row * kHeadDim) = vc[u];
      }
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
      unpack_v<KV>(vc[u], vf);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = fmaf(p, vf[i], acc[i]);
    }
    m_run = m_new;
    if (more) {
      if (!RSWA_DECODE_PREFETCH) load(rb + STEP, kn, vn);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kc[u] = kn[u];
        vc[u] = vn[u];
      }
    }
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
    if (direct) {
      store_out(reinterpret_cast<OUT*>(a.out) + bh * kHeadDim + tid, num / lsum);
    } else {
      a.ws_acc[slot * kHeadDim + tid] = num;
      if (tid == 0) a.ws_ml[slot] = make_float2(M, lsum);
    }
  }
  __syncthreads();
}

template <typename KV, typename OUT, int U>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];
  __shared__ float s_m[kMaxGroups], s_l[kMaxGroups];
  __shared__ float s_acc[kMaxGroups * kHeadDim];
  int64_t* s_cum = reinterpret_cast<int64_t*>(s_dyn);
  int* s_len = reinterpret_cast<int*>(s_cum + a.batch + 1);
  int* s_new = s_len + a.batch;
  build_work_table(a, s_len, s_new, s_cum);
  const int H = a.heads;
  const int64_t total = s_cum[a.batch];

  if (a.aligned) {
    const int s = blockIdx.x;
    const int b = s / H, h = s - (s / H) * H;
    if (b >= a.batch || s_len[b] == 0) return;
    decode_range<KV, OUT, U>(a, b, h, 0, s_len[b], s_new[b], true, 0, s_m, s_l, s_acc);
    return;
  }

  const int64_t W = piece_rows(a, total);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    for (int b = 0; b <= a.batch; ++b) a.ws_cum[b] = s_cum[b];
    a.ws_cum[a.batch + 1] = W;
  }
  int64_t pos = (int64_t)blockIdx.x * W;
  const int64_t end = min(pos + W, total);
  while (pos < end) {
    int lo = 0, hi = a.batch - 1;  // last b with s_cum[b] <= pos
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_cum[mid] <= pos) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int L = s_len[b];
    const int64_t off = pos - s_cum[b];
    const int h = (int)(off / L);
    const int r0 = (int)(off - (int64_t)h * L);
    const int r1 = (int)min((int64_t)L, r0 + (end - pos));
    const int s = b * H + h;
    const int64_t A = s_cum[b] + (int64_t)h * L;
    const bool direct = A / W == (A + L - 1) / W;
    decode_range<KV, OUT, U>(a, b, h, r0, r1, s_new[b], direct, (int64_t)blockIdx.x + s, s_m,
                             s_l, s_acc);
    pos += r1 - r0;
  }
}

// One workgroup per (b, h): combine the partials of a range split over several pieces.
template <typename OUT>
__global__ __launch_bounds__(kHeadDim) void decode_merge_kernel(DecodeArgs a) {
  __shared__ float s_w[kMergeChunk], s_l[kMergeChunk];
  __shared__ float s_red[kHeadDim / kWave];
  const int s = blockIdx.x;
  const int b = s / a.heads, h = s - (s / a.heads) * a.heads;
  const int64_t c0 = a.ws_cum[b], c1 = a.ws_cum[b + 1];
  const int64_t L = (c1 - c0) / a.heads;
  if (L == 0) return;
  const int64_t W = a.ws_cum[a.batch + 1];
  const int64_t A = c0 + h * L;
  const int64_t f = A / W, l = (A + L - 1) / W;
  if (f == l) return;  // written directly by the decode kernel
  merge_range<OUT>(a, s, f, (int)(l - f + 1), s_w, s_l, s_red);
}

#ifndef RSWA_DECODE_ROWS
#define RSWA_DECODE_ROWS 2
#endif
constexpr int kRowsPerLane = RSWA_DECODE_ROWS;  // U: rows each lane group loads per tile

template <typename KV, typename OUT>
hipError_t launch_typed(const DecodeArgs& a, int grid, bool need_merge, hipStream_t s) {
  const size_t smem = decode_lds_bytes(a.batch);
  if (grid > 0) {
    hipLaunchKernelGGL((decode_kernel<KV, OUT, kRowsPerLane>), dim3(grid), dim3(kThreads), smem,
                       s, a);
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

template <typename KV, typename OUT>
int occupancy_typed(int batch) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<KV, OUT, kRowsPerLane>,
                                                   kThreads, decode_lds_bytes(batch)) != hipSuccess)
    return 1;
  return n > 0 ? n : 1;
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

size_t decode_lds_bytes(int batch) {
  return (size_t)(batch + 1) * sizeof(int64_t) + (size_t)2 * batch * sizeof(int);
}

int decode_blocks_per_cu(int kv_f32, int out_f32, int batch) {
  if (kv_f32)
    return out_f32 ? occupancy_typed<float, float>(batch) : occupancy_typed<float, uint16_t>(batch);
  return out_f32 ? occupancy_typed<uint16_t, float>(batch)
                 : occupancy_typed<uint16_t, uint16_t>(batch);
}

}  // namespace rswa
