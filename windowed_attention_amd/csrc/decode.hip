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
//  * split: fewer equal ranges are each cut into k equal pieces (every piece then holds rows of
//    one range only and publishes its partial once, at its end), merged like the stream-K ranges
//    below;
//  * stream-K: the concatenation of all (b, h) key ranges is cut into equal contiguous pieces, one
//    per resident workgroup, so every workgroup streams the same number of rows (no tail round,
//    balanced for ragged batches). A piece may cover parts of several ranges; a range split over
//    several pieces leaves float32 partials (max, sum, numerator[128]), and the last of its
//    pieces to finish merges them in the same launch:
//      o = sum_s 2^(M_s - M) A_s / sum_s 2^(M_s - M) l_s,   M = max_s M_s.
//
// The in-launch merge. A piece publishes its partial with device-scope (agent) stores, waits until
// they are complete, then adds one to the range's counter with a device-scope atomic; the piece
// that brings the counter to the range's piece count reads every partial with device-scope loads,
// writes the output and resets the counter for the next launch. Device-scope stores and loads
// reach the point where the XCDs' L2 caches are coherent, so no L2 write-back or invalidate (what
// a release / acquire fence at device scope costs, once per workgroup) is needed; measured, those
// fences made the step several times slower, and a separate merge launch costs a kernel dispatch
// (about 2.7 us back to back on MI355X) plus a memory round trip for its plan.
//
// Inside a piece. A row of K or V is 256 B (bf16) or 512 B (fp32): 16 or 32 lanes each load 16 B of
// it, so a wave streams 4 (bf16) or 2 (fp32) rows per load instruction, 1 KiB contiguous. Two
// register sets alternate: the loads of the next tile are issued before the current tile is
// reduced, always (rows clamped to the range; past its end they re-read its last row, which the
// caches hold), so the compiler's waits leave them in flight. Each lane group keeps its own
// float32 online-softmax state (running max in the log2 domain, running sum, 8 or 4 output dims);
// q.k partial dot products are summed across the group with DPP row operations. At the end of a
// range the group states are merged through LDS.
//
// Streamed steps. When a step's live rows exceed the last-level cache (the host decides from the
// row counts; paged caches excepted), none of them is still cached at the next step, so a second
// copy of the tile loop reads them with non-temporal loads, two tiles a round, both waited for
// before both are reduced (fewer requests in flight per wave), and the host plans such a step over
// three workgroups per CU instead of four.
//
// Fused append (K1 inside K2). When the launch carries the new k/v rows, the new row's slot
// r = m_b + (t_b mod n_b) (or m_b + t_b) is part of the live range after the append; the lane group
// that meets this row in its piece takes k/v from the input instead of the cache and writes them
// into the slot, so no other workgroup reads the slot during the launch and the evicted output is
// never seen.
#include "device.h"
#include "kernels.h"
#include "plan.h"

namespace rswa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxGroups = kWaves * 4;  // bf16: 4 row groups per wave
constexpr float kLazy = 8.f;            // log2-domain slack before the reference max moves

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

// Whether the launch has the plan of sequences that share m, capacity and step count, and that
// count: passed by the host (uni_t >= 0), or, in a captured step, read from the counters.
__device__ __forceinline__ bool uni_plan(const DecodeArgs& a) {
  return a.uni_t >= 0 || a.uni_t == kUniFromCounters;
}
__device__ __forceinline__ int uni_count(const DecodeArgs& a) {
  return a.uni_t >= 0 ? a.uni_t : __builtin_amdgcn_readfirstlane(a.steps_in[0]);
}

__device__ __forceinline__ SeqState seq_state(const DecodeArgs& a, int b) {
  SeqState st;
  const bool uni = uni_plan(a);
  const bool act = uni || !a.active || a.active[b];
  st.t = uni ? uni_count(a) : a.steps_in[b];
  const int cap = uni ? a.uni_cap : a.meta.cap[b];
  st.app = act && a.k_new != nullptr && (!a.full_causal || st.t < cap);
  const int t_after = st.app ? st.t + 1 : st.t;
  st.L = act ? (uni ? a.uni_m : a.meta.prefix_len[b]) + min(t_after, cap) : 0;
  return st;
}

// Work table in LDS: s_len[b] = live rows, s_new[b] = cache row of this launch's new k/v (or -1),
// s_cum[b] = sum over b' < b of H * L_b' (int64). Block 0 also advances the step counters.
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
      const bool uni = uni_plan(a);
      const int m = uni ? a.uni_m : a.meta.prefix_len[b];
      const int cap = uni ? a.uni_cap : a.meta.cap[b];
      if (st.app) rnew = a.full_causal ? m + st.t : m + st.t % cap;
      s_new[b] = rnew;
      if (blockIdx.x == 0) {
        if (a.steps_out) a.steps_out[b] = st.app ? st.t + 1 : st.t;
        if (a.k_new && a.full_causal && (!a.active || a.active[b]) && st.t >= cap) *a.meta.err = 1;
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

// Global-memory load (the explicit address space keeps it a global load where the pointer has
// been through readfirstlane, which hides where it points from the compiler).
typedef const __attribute__((address_space(1))) u32x4* gptr16;
__device__ __forceinline__ u32x4 ld16(const void* p) { return *(gptr16)p; }
// Non-temporal loads (cache policy bit `nt`): the lines are not kept in the caches for reuse. A
// step that reads more than the last-level cache holds finds none of its rows there at the next
// step anyway, and streaming them avoids evicting what does get reused. They are issued as buffer
// loads from a resource over one wave's tile (base = the tile's first row, in scalar registers),
// a different instruction from the plain global load, so the compiler cannot merge the two
// variants of a tile load into one (merging drops the non-temporal mark).
constexpr int kCachePolicyNT = 2;            // aux bit of the buffer-load builtin: nt
constexpr int kBufferRsrcWord3 = 0x00020000; // raw (unformatted) 32-bit data, no swizzle
// A pointer that is the same in every lane, passed through readfirstlane so that the compiler
// sees it and keeps it (and what is computed from it) in scalar registers; a buffer resource built
// from a value it cannot prove uniform makes it wrap every load in a loop over lane values.
template <typename T>
__device__ __forceinline__ T* wave_uniform(T* ptr) {
  const uint64_t p = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(wave_uniform(const_cast<void*>(base)), (short)0, bytes,
                                           kBufferRsrcWord3);
}
struct Plain { static constexpr bool value = false; };
struct Streamed { static constexpr bool value = true; };
__device__ __forceinline__ u32x4 ld16_stream(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0,
                                                                          kCachePolicyNT));
}

// Device-scope (agent) accesses of the merge workspace: coherent across the XCDs' L2 caches
// without a cache write-back or invalidate.
__device__ __forceinline__ void st_dev(float* p, float x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this thread's stores are complete (device-scope stores: visible to every XCD).
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Combine the np partials of range s stored at workspace slots f + s .. f + s + np - 1 and write
// the output; threads [0, 128) hold one output dim each. Partial (max, sum) pairs sit at
// ws_ml[2 slot], ws_ml[2 slot + 1]. Every partial of the range is requested at once (up to
// kMergeFast), so the merge waits for memory once instead of once per piece.
constexpr int kMergeChunk = kHeadDim;
constexpr int kMergeFast = 16;

template <typename OUT>
__device__ __forceinline__ void merge_range(const DecodeArgs& a, int64_t s, int64_t f, int np,
                                            float* s_w, float* s_l, float* s_red) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  constexpr int NW = kHeadDim / kWave;
  const bool worker = tid < kHeadDim;
  const float* ml = a.ws_ml + 2 * (f + s);
  const float* acc = a.ws_acc + (f + s) * kHeadDim + (worker ? tid : 0);
  float M = kNegBig;
  if (np <= kMergeFast) {
    const float pm = tid < np ? ld_dev(ml + 2 * tid) : kNegBig;
    const float pl = tid < np ? ld_dev(ml + 2 * tid + 1) : 0.f;
    float x[kMergeFast];
#pragma unroll
    for (int i = 0; i < kMergeFast; ++i) x[i] = (worker && i < np) ? ld_dev(acc + (int64_t)i * kHeadDim) : 0.f;
    M = pm;
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    if (lane == 0 && wave < NW) s_red[wave] = M;
    __syncthreads();
    M = s_red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_red[w]);
    if (tid < np) {
      s_w[tid] = fast_exp2(pm - M);
      s_l[tid] = pl;
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
    for (int i = tid; i < np; i += kHeadDim) M = fmaxf(M, ld_dev(ml + 2 * i));
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
      s_w[tid] = fast_exp2(ld_dev(ml + 2 * (c + tid)) - M);
      s_l[tid] = ld_dev(ml + 2 * (c + tid) + 1);
    }
    __syncthreads();
    if (worker) {
      int i = 0;
      for (; i + 4 <= n; i += 4) {
        const float x0 = ld_dev(acc + (int64_t)(c + i) * kHeadDim);
        const float x1 = ld_dev(acc + (int64_t)(c + i + 1) * kHeadDim);
        const float x2 = ld_dev(acc + (int64_t)(c + i + 2) * kHeadDim);
        const float x3 = ld_dev(acc + (int64_t)(c + i + 3) * kHeadDim);
        num = fmaf(x0, s_w[i], num);
        num = fmaf(x1, s_w[i + 1], num);
        num = fmaf(x2, s_w[i + 2], num);
        num = fmaf(x3, s_w[i + 3], num);
      }
      for (; i < n; ++i) num = fmaf(ld_dev(acc + (int64_t)(c + i) * kHeadDim), s_w[i], num);
      for (int j = 0; j < n; ++j) lsum = fmaf(s_l[j], s_w[j], lsum);
    }
  }
  if (worker) store_out(reinterpret_cast<OUT*>(a.out) + s * kHeadDim + tid, num / lsum);
  __syncthreads();
}

// The workgroups that share a CU (three or four) do not progress evenly: the oldest waves win the
// issue arbitration, so some pieces finish early and the rest then run with a fraction of the CU's
// waves in flight. A wave lowers its issue priority as its piece progresses (done of total rows), which
// hands issue slots to the pieces that are behind.
__device__ __forceinline__ void yield_by_progress(int64_t done, int64_t total) {
  const int64_t lvl = (4 * done) / total;
  if (lvl <= 0) asm volatile("s_setprio 3");
  else if (lvl == 1) asm volatile("s_setprio 2");
  else if (lvl == 2) asm volatile("s_setprio 1");
  else asm volatile("s_setprio 0");
}

// Stream rows [r0, r1) of range (b, h); finish with the group merge through LDS, then either the
// output (the range is not split) or a partial in workspace slot `slot`, published at device
// scope. Returns (in every thread) whether this piece is the last of the range's np pieces to
// publish, in which case the caller merges.
template <typename KV, typename OUT, int U>
__device__ __forceinline__ bool decode_range(const DecodeArgs& a, int b, int h, int r0, int r1,
                                             int rnew, bool direct, int64_t slot, int np,
                                             float* s_m, float* s_l, float* s_acc, int* s_flag,
                                             int64_t done0, int64_t piece) {
  constexpr int VEC = Lanes<KV>::VEC, GL = Lanes<KV>::GL, G = kWave / GL, NG = kWaves * G;
  constexpr int STEP = kWaves * G * U;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // tile decisions are scalar
  const int g = lane / GL, li = lane % GL;
  const int H = a.heads;
  const bool uni = uni_plan(a);
  const int64_t R = uni ? a.uni_rows : a.meta.rows[b];
  const int m = uni ? a.uni_m : a.meta.prefix_len[b];
  // Cache row r lives at Kh + r * D; with a paged prefix the storage starts at row m, and rows
  // r < m are pool rows found through the page table (one 4-byte lookup per row and group).
  const bool paged = a.meta.table != nullptr;
  const int64_t shift = paged ? m : 0;
  KV* seq = reinterpret_cast<KV*>(a.storage) +
            (uni ? (int64_t)b * 2 * H * R * kHeadDim : a.meta.seq_off[b]);
  KV* Kh = seq + ((int64_t)h * R - shift) * kHeadDim;
  KV* Vh = seq + ((int64_t)(H + h) * R - shift) * kHeadDim;
  KV* Kp = Kh + li * VEC;
  KV* Vp = Vh + li * VEC;
  const int lane_el = g * kHeadDim + li * VEC;  // this lane's 16 B in a tile's first row group
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
  const float c = a.scale_log2;

  // Softmax state per lane group, log2 domain, against a lazily moved reference max: the state is
  // rescaled only when a score passes the reference by kLazy, so a probability never exceeds
  // 2^kLazy and most tiles skip the rescale (a scalar branch on a wave ballot).
  float m_ref = kNegBig, m_thr = kNegBig, l_run = 0.f;
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;

  // The new row (fused append): its k / v come from the input, loaded once into registers; the
  // tile that holds it swaps them in and writes them into the ring slot.
  // Only the piece whose rows hold the new row touches it (a tile running past the piece's end
  // may reach the next piece's new row; that row is masked there).
  u32x4 knew = {0u, 0u, 0u, 0u}, vnew = {0u, 0u, 0u, 0u};
  const int rn = (rnew >= r0 && rnew < r1) ? rnew : -1;
  if (rn >= 0) {
    knew = ld16(kin);
    vnew = ld16(vin);
  }

  auto reduce = [&](int base, u32x4* kc, u32x4* vc) {
    if ((unsigned)(rn - base) < (unsigned)(G * U)) {  // this tile holds the new row
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = base + u * G + g;
        if (row == rn) {
          kc[u] = knew;
          vc[u] = vnew;
          *reinterpret_cast<u32x4*>(Kp + (int64_t)row * kHeadDim) = knew;
          *reinterpret_cast<u32x4*>(Vp + (int64_t)row * kHeadDim) = vnew;
        }
      }
    }
    float d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) d[u] = group_sum<KV>(partial_dot<KV>(qv, kc[u]));
    if (base + G * U > r1) {  // the range ends inside this tile: rows past it do not count, and
                              // their values (whatever the memory holds) must not reach acc
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (base + u * G + g >= r1) {
          d[u] = -INFINITY;
          vc[u] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    float mx = d[0];
#pragma unroll
    for (int u = 1; u < U; ++u) mx = fmaxf(mx, d[u]);
    const float cand = mx * c;
    if (__builtin_amdgcn_ballot_w64(cand > m_thr)) {
      const float m_new = fmaxf(m_ref, cand);
      const float alpha = fast_exp2(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] *= alpha;
      m_ref = m_new;
      m_thr = m_new + kLazy;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = fast_exp2(fmaf(d[u], c, -m_ref));
      l_run += p;
      float vf[VEC];
      unpack_v<KV>(vc[u], vf);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = fmaf(p, vf[i], acc[i]);
    }
  };

  int rb = r0 + wave * (G * U);
  u32x4 ka[U], va[U], kb[U], vb[U];
  if (paged) {
    // Prefix rows looked up in the page table (a tile may straddle the prefix end): a plain loop.
    const int pend = min(m, r1);
    for (; rb < pend; rb += STEP) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int rr = min(rb + u * G + g, r1 - 1);
        if (rr < m) {
          const int64_t pr = (int64_t)tab[rr] * pool_stride;
          ka[u] = ld16(PKp + pr);
          va[u] = ld16(PVp + pr);
        } else {
          ka[u] = ld16(Kp + (int64_t)rr * kHeadDim);
          va[u] = ld16(Vp + (int64_t)rr * kHeadDim);
        }
      }
      reduce(rb, ka, va);
    }
  }
  if (rb < r1) {
    // Cache rows: a scalar tile base plus fixed lane offsets, no clamps. The rows of the last tile
    // past the range belong to the next range, or to the storage's tail bytes, and are masked.
    // Two register sets alternate, and the tile after this wave's last is its last again (the
    // caches hold it), so every load can be issued a tile ahead without a condition.
    const int last = rb + ((r1 - 1 - rb) / STEP) * STEP;
    // Streamed (non-temporal) loads: a buffer resource over the wave's tile of K and of V. The loop
    // is compiled once per load kind and the launch picks one, so no tile tests the choice.
    constexpr int RB = kHeadDim * (int)sizeof(KV);  // bytes per row
    const int lane_b = lane_el * (int)sizeof(KV);
    // The tile loop addresses rows from scalar bases (the same in every lane).
    const KV* const Ks = wave_uniform(Kh);
    const KV* const Vs = wave_uniform(Vh);
    auto tile_loop = [&](auto kind) {
      auto load = [&](int base, u32x4* kr, u32x4* vr) {
        const KV* kt = Ks + (int64_t)base * kHeadDim;
        const KV* vt = Vs + (int64_t)base * kHeadDim;
        if constexpr (decltype(kind)::value) {
          const __amdgpu_buffer_rsrc_t krs = tile_rsrc(kt, U * G * RB);
          const __amdgpu_buffer_rsrc_t vrs = tile_rsrc(vt, U * G * RB);
#pragma unroll
          for (int u = 0; u < U; ++u) {
            kr[u] = ld16_stream(krs, lane_b + u * G * RB);
            vr[u] = ld16_stream(vrs, lane_b + u * G * RB);
          }
        } else {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            kr[u] = ld16(kt + lane_el + u * G * kHeadDim);
            vr[u] = ld16(vt + lane_el + u * G * kHeadDim);
          }
        }
      };
      if constexpr (decltype(kind)::value) {
        // Two tiles per round, both loaded and waited for, then both reduced: a wave keeps fewer
        // requests in flight than in the pipelined loop below, and the streamed step runs faster
        // so (346 MB: 56.2 us, vs 56.9 waiting for one tile's loads a round and 58.4 pipelined).
        for (;;) {
          load(rb, ka, va);
          load(min(rb + STEP, last), kb, vb);
          wait_loads();
          reduce(rb, ka, va);
          if (rb + STEP > last) break;
          reduce(rb + STEP, kb, vb);
          rb += 2 * STEP;
          if (rb > last) break;
          yield_by_progress(done0 + (rb - r0), piece);
        }
      } else {
        load(rb, ka, va);
        for (;;) {
          load(min(rb + STEP, last), kb, vb);
          reduce(rb, ka, va);
          rb += STEP;
          if (rb > last) break;
          load(min(rb + STEP, last), ka, va);
          reduce(rb, kb, vb);
          rb += STEP;
          if (rb > last) break;
          yield_by_progress(done0 + (rb - r0), piece);
        }
      }
    };
    if (a.stream_loads)
      tile_loop(Streamed{});
    else
      tile_loop(Plain{});
  }

  const int gid = wave * G + g;
#pragma unroll
  for (int i = 0; i < VEC; ++i) s_acc[gid * kHeadDim + li * VEC + i] = acc[i];
  if (li == 0) {
    s_m[gid] = m_ref;
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
      st_dev(a.ws_acc + slot * kHeadDim + tid, num);
      if (tid == 0) {
        st_dev(a.ws_ml + 2 * slot, M);
        st_dev(a.ws_ml + 2 * slot + 1, lsum);
      }
      wait_stores();
    }
  }
  if (direct) {
    __syncthreads();
    return false;
  }
  __syncthreads();  // every store of the partial is complete
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(a.ws_cnt + bh, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == np - 1;
    if (last) __hip_atomic_store(a.ws_cnt + bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = last;
  }
  __syncthreads();
  return *s_flag != 0;
}

template <typename KV, typename OUT, int U>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];
  __shared__ float s_m[kMaxGroups], s_l[kMaxGroups];
  __shared__ float s_acc[kMaxGroups * kHeadDim];
  __shared__ float s_w[kMergeChunk], s_lw[kMergeChunk];
  __shared__ float s_red[kHeadDim / kWave];
  __shared__ int s_flag;
  int64_t* s_cum = reinterpret_cast<int64_t*>(s_dyn);
  int* s_len = reinterpret_cast<int*>(s_cum + a.batch + 1);
  int* s_new = s_len + a.batch;
  const int H = a.heads;

  if (uni_plan(a) && (a.aligned || a.split > 1)) {
    // Host-known plan over equal ranges: every sequence has the same live rows and new-row slot,
    // so no work table (and none of its barriers) is needed; block 0 advances the counters.
    const SeqState st = seq_state(a, 0);
    const int rnew = st.app ? (a.full_causal ? a.uni_m + st.t : a.uni_m + st.t % a.uni_cap) : -1;
    if (blockIdx.x == 0)
      for (int b = threadIdx.x; b < a.batch; b += kThreads) {
        if (a.steps_out) a.steps_out[b] = st.app ? st.t + 1 : st.t;
        if (a.k_new && a.full_causal && st.t >= a.uni_cap) *a.meta.err = 1;
      }
    if (st.L == 0) return;
    if (a.aligned) {
      const int s = blockIdx.x;
      const int b = s / H, h = s - b * H;
      if (b >= a.batch) return;
      decode_range<KV, OUT, U>(a, b, h, 0, st.L, rnew, true, 0, 1, s_m, s_l, s_acc, &s_flag, 0,
                               st.L);
      return;
    }
    const int k = a.split;
    const int s = blockIdx.x / k, i = blockIdx.x - s * k;
    const int b = s / H, h = s - b * H;
    if (b >= a.batch) return;
    const int r0 = (int)((int64_t)st.L * i / k), r1 = (int)((int64_t)st.L * (i + 1) / k);
    if (decode_range<KV, OUT, U>(a, b, h, r0, r1, rnew, false, (int64_t)blockIdx.x + s, k, s_m,
                                 s_l, s_acc, &s_flag, 0, max(r1 - r0, 1)))
      merge_range<OUT>(a, s, (int64_t)s * k, k, s_w, s_lw, s_red);
    return;
  }

  build_work_table(a, s_len, s_new, s_cum);
  const int64_t total = s_cum[a.batch];

  if (a.aligned) {
    const int s = blockIdx.x;
    const int b = s / H, h = s - (s / H) * H;
    if (b >= a.batch || s_len[b] == 0) return;
    decode_range<KV, OUT, U>(a, b, h, 0, s_len[b], s_new[b], true, 0, 1, s_m, s_l, s_acc,
                             &s_flag, 0, s_len[b]);
    return;
  }

  if (a.split > 1) {  // piece i of range s: rows [i L / k, (i + 1) L / k)
    const int k = a.split;
    const int s = blockIdx.x / k, i = blockIdx.x - s * k;
    const int b = s / H, h = s - (s / H) * H;
    if (b >= a.batch || s_len[b] == 0) return;
    const int L = s_len[b];
    const int r0 = (int)((int64_t)L * i / k), r1 = (int)((int64_t)L * (i + 1) / k);
    if (decode_range<KV, OUT, U>(a, b, h, r0, r1, s_new[b], false, (int64_t)blockIdx.x + s, k,
                                 s_m, s_l, s_acc, &s_flag, 0, max(r1 - r0, 1)))
      merge_range<OUT>(a, s, (int64_t)s * k, k, s_w, s_lw, s_red);
    return;
  }

  const int64_t W = piece_rows(a, total);
  const int64_t pos0 = (int64_t)blockIdx.x * W;
  int64_t pos = pos0;
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
    const int64_t f = A / W, l = (A + L - 1) / W;  // pieces that hold rows of this range
    const bool direct = f == l;
    if (decode_range<KV, OUT, U>(a, b, h, r0, r1, s_new[b], direct, (int64_t)blockIdx.x + s,
                                 (int)(l - f + 1), s_m, s_l, s_acc, &s_flag, pos - pos0, W))
      merge_range<OUT>(a, s, f, (int)(l - f + 1), s_w, s_lw, s_red);
    pos += r1 - r0;
  }
}

#ifndef RSWA_DECODE_ROWS
#define RSWA_DECODE_ROWS 2
#endif
constexpr int kRowsPerLane = RSWA_DECODE_ROWS;  // U: rows each lane group loads per tile
// A tile is loaded whole, so the last tile of the storage's last range may read up to
// (rows per wave tile - 1) rows past its final row; the storage's unused tail must hold them.
template <typename KV>
constexpr uint64_t tile_overread_bytes() {
  return (uint64_t)(kWave / Lanes<KV>::GL * kRowsPerLane - 1) * kHeadDim * sizeof(KV);
}
static_assert(tile_overread_bytes<uint16_t>() <= kStorageTailBytes &&
                  tile_overread_bytes<float>() <= kStorageTailBytes,
              "decode tiles would read past the storage tail");

template <typename KV, typename OUT>
hipError_t launch_typed(const DecodeArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((decode_kernel<KV, OUT, kRowsPerLane>), dim3(grid), dim3(kThreads),
                     decode_lds_bytes(a.batch), s, a);
  return hipGetLastError();
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
                         hipStream_t s) {
  if (kv_f32) {
    return out_f32 ? launch_typed<float, float>(a, grid_blocks, s)
                   : launch_typed<float, uint16_t>(a, grid_blocks, s);
  }
  return out_f32 ? launch_typed<uint16_t, float>(a, grid_blocks, s)
                 : launch_typed<uint16_t, uint16_t>(a, grid_blocks, s);
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
