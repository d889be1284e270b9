// K3: R-SWA-masked prefill / teacher-forced attention on bf16 MFMA (gfx950).
//
// Mask (deep dive "Unlimited-OCR", N(t) code block; GeekNews "Unlimited OCR", R-SWA section and the
// training section's packed multi-page sequences): in a sequence of S tokens whose first m are the
// reference prefix, query p sees
//   prefix key k < m: always (or only k <= p for prefix queries when the prefix is causal);
//   output key k >= m: iff k <= p and p - k < n (its own window of n outputs, itself included).
// A query tile therefore visits two key segments only: the prefix [0, m) and the window
// [max(m, q_first - n + 1), q_last]; every other key tile is skipped without being loaded. Element
// masks are applied only on tiles that need them (the prefix's ragged last tile, the causal-prefix
// diagonal, and the window tiles).
//
// Tiling. A workgroup of RSWA_PF_WAVES waves (8: 512 threads, two waves per SIMD) owns 32 queries
// per wave of one (sequence, head).
// Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the accumulator puts one
// query per lane (lane % 32) and 16 of the block's 32 keys in that lane's registers, so the softmax
// max/sum over keys is in-lane plus one exchange with lane ^ 32. The output is also formed
// transposed, O^T = V^T P^T: the score accumulator registers, rounded to bf16, are already the B
// operand of the second MFMA (the key order inside a 16-key step is a permutation that the V^T
// operand follows), so P never leaves registers. K and V tiles (64 keys x 128) are
// double-buffered in LDS, both row-major (rows padded against bank conflicts), and loaded two
// tiles ahead; the V^T operand comes out of gfx950's transposing LDS read, so V needs no transpose
// on the way in. Q stays in registers for the whole key loop. Softmax runs in the log2 domain in
// float32 with a lazily moved reference max; P is rounded to bf16 for the PV product and the
// output is normalised by the float32 row sum. With a non-null lse the natural log-sum-exp of
// each query's scaled scores is written too (the training pass needs it).
#include "kernels.h"
#include "mfma.h"

namespace rswa {
namespace {

#ifndef RSWA_PF_SCHED
#define RSWA_PF_SCHED 4  // > 0: K-fragment LDS reads kept ahead of the score MFMAs
#endif
#ifndef RSWA_PF_WAVES
#define RSWA_PF_WAVES 8  // waves per workgroup (each owns QB x 32 queries)
#endif
constexpr int kWavesPF = RSWA_PF_WAVES;
constexpr int kThreads = 64 * kWavesPF;
constexpr int kKeysPerThread = 64 * 16 / kThreads;  // a 64-key tile is 64 x 16 pieces of 16 B
constexpr int BN = 64;                  // keys per tile
#ifndef RSWA_PF_KPAD
#define RSWA_PF_KPAD 8   // bf16 pad per K row (bank spread of the 16-byte operand reads)
#endif
#ifndef RSWA_PF_VPAD
#define RSWA_PF_VPAD 32  // bf16 pad per V row (bank spread of the transposing reads)
#endif
constexpr int KSTR = kHeadDim + RSWA_PF_KPAD;  // K tile row stride (bf16)
constexpr int VSTR = kHeadDim + RSWA_PF_VPAD;  // V tile row stride (bf16)
constexpr int K_TILE = BN * KSTR;              // bf16 elements per K buffer
constexpr int V_TILE = BN * VSTR;              // bf16 elements per V buffer
constexpr float kLazy = 8.f;            // log2-domain slack before the reference max moves

struct TileSched {
  int n_pre;   // tiles over the prefix segment [0, pre_end)
  int pre_end;
  int ws;      // first key of the window segment
  int ntiles;
  __device__ __forceinline__ int start(int j) const { return j < n_pre ? j * BN : ws + (j - n_pre) * BN; }
};

// Global -> registers: thread t loads kKeysPerThread consecutive keys x 8 dims of K and of V.
__device__ __forceinline__ void load_tile(u32x4 (&rk)[kKeysPerThread], u32x4 (&rv)[kKeysPerThread],
                                          const uint16_t* kbase, const uint16_t* vbase,
                                          int64_t row_stride, int k0, int kmax) {
  const int t = threadIdx.x;
  const int c = t & 15, kg = t >> 4;
#pragma unroll
  for (int u = 0; u < kKeysPerThread; ++u) {
    const int key = min(k0 + kg * kKeysPerThread + u, kmax);
    rk[u] = *reinterpret_cast<const u32x4*>(kbase + key * row_stride + c * 8);
    rv[u] = *reinterpret_cast<const u32x4*>(vbase + key * row_stride + c * 8);
  }
}

// Registers -> LDS: K and V tiles both row-major (key rows of 128 dims), 16-byte stores.
__device__ __forceinline__ void store_tile(const u32x4 (&rk)[kKeysPerThread],
                                           const u32x4 (&rv)[kKeysPerThread], uint16_t* sk,
                                           uint16_t* sv) {
  const int t = threadIdx.x;
  const int c = t & 15, kg = t >> 4;
#pragma unroll
  for (int u = 0; u < kKeysPerThread; ++u) {
    *reinterpret_cast<u32x4*>(sk + (kg * kKeysPerThread + u) * KSTR + c * 8) = rk[u];
    *reinterpret_cast<u32x4*>(sv + (kg * kKeysPerThread + u) * VSTR + c * 8) = rv[u];
  }
}

// QB query blocks of 32 per wave: every K / V^T fragment read from LDS feeds QB MFMAs.
template <typename OUT, int QB>
__global__ __launch_bounds__(kThreads, (QB == 1 ? 8 : 4) / kWavesPF) void prefill_kernel(
    PrefillArgs a) {
  constexpr int BMQ = kWavesPF * 32 * QB;  // queries per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t sK[2 * K_TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2 * V_TILE];

  const int s = blockIdx.z, h = blockIdx.y;
  const int cu0 = a.cu_seqlens[s];
  const int S = a.cu_seqlens[s + 1] - cu0;
  const int q0 = blockIdx.x * BMQ;
  if (q0 >= S) return;
  const int q1 = min(q0 + BMQ, S);
  const int m = a.prefix_len[s];
  const int n = a.window[s];
  const bool pc = a.prefix_causal != 0;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, half = lane >> 5;
  const int64_t rs = (int64_t)a.heads * kHeadDim;  // token row stride (elements)
  const uint16_t* qbase = a.q + ((int64_t)cu0 * a.heads + h) * kHeadDim;
  const uint16_t* kbase = a.k + ((int64_t)cu0 * a.heads + h) * kHeadDim;
  const uint16_t* vbase = a.v + ((int64_t)cu0 * a.heads + h) * kHeadDim;

  // this lane's queries (one per query block) and their Q^T operands (8 d-steps of 16)
  int p[QB];
  u32x4 qf[QB][8];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    p[qb] = q0 + (wave * QB + qb) * 32 + lq;
    const int pq = min(p[qb], S - 1);
#pragma unroll
    for (int st = 0; st < 8; ++st)
      qf[qb][st] = *reinterpret_cast<const u32x4*>(qbase + pq * rs + st * 16 + half * 8);
  }

  // key tiles: the prefix segment, then the output window segment
  TileSched ts;
  ts.pre_end = (pc && q1 <= m) ? q1 : m;
  ts.n_pre = (ts.pre_end + BN - 1) / BN;
  int n_win = 0;
  ts.ws = 0;
  if (q1 > m) {
    ts.ws = max(m, max(q0, m) - n + 1);
    n_win = (q1 - ts.ws + BN - 1) / BN;
  }
  ts.ntiles = ts.n_pre + n_win;

  // visible key interval of each query in each segment: prefix [0, pre_hi], window [win_lo, p]
  int pre_hi[QB], win_lo[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    pre_hi[qb] = (pc && p[qb] < m) ? min(p[qb], m - 1) : m - 1;
    win_lo[qb] = p[qb] >= m ? max(m, p[qb] - n + 1) : p[qb] + 1;  // empty for prefix queries
  }

  const float c = a.scale_log2;
  float m_run[QB], l_run[QB];
  floatx16 o[QB][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = kNegBig;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.f;
  }

  // Global -> register loads run two tiles ahead (register sets A and B alternate), so a tile's
  // loads have two tiles of compute to arrive; LDS holds two tiles (being read / being written).
  u32x4 ka_[kKeysPerThread], va_[kKeysPerThread], kb_[kKeysPerThread], vb_[kKeysPerThread];
  load_tile(ka_, va_, kbase, vbase, rs, ts.start(0), S - 1);
  store_tile(ka_, va_, sK, sV);
  if (ts.ntiles > 1) load_tile(ka_, va_, kbase, vbase, rs, ts.start(1), S - 1);
  __syncthreads();

  // one tile: S^T, mask, softmax and PV from LDS buffer `buf`
  auto tile = [&](int j, int buf) {
    const uint16_t* sk = sK + buf * K_TILE;
    const uint16_t* sv = sV + buf * V_TILE;
    const int k0 = ts.start(j);
    const bool is_pre = j < ts.n_pre;

    // S^T = K Q^T for two 32-key blocks; each K fragment feeds QB MFMAs
    floatx16 sacc[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[qb][kb][r] = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const u32x4 ka =
            *reinterpret_cast<const u32x4*>(sk + (kb * 32 + lq) * KSTR + st * 16 + half * 8);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[qb][kb] = mfma32(ka, qf[qb][st], sacc[qb][kb]);
      }
#if RSWA_PF_SCHED
    // keep RSWA_PF_SCHED K-fragment reads in flight ahead of the score MFMA chain
    __builtin_amdgcn_sched_group_barrier(0x100, RSWA_PF_SCHED, 0);
#pragma unroll
    for (int i = 0; i < 16 - RSWA_PF_SCHED; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, QB * RSWA_PF_SCHED, 0);
#endif

    // element mask (branch-free interval test) where the tile is not fully visible
    const bool need_mask = is_pre ? (k0 + BN > m || (pc && q0 < m && k0 + BN - 1 > q0)) : true;
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int lo = is_pre ? 0 : win_lo[qb];
        const int hi = is_pre ? pre_hi[qb] : p[qb];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int k = k0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            sacc[qb][kb][r] = (k >= lo && k <= hi) ? sacc[qb][kb][r] : -INFINITY;
          }
      }
    }

    // Online softmax (log2 domain), one query per lane, keys split across lane and lane ^ 32,
    // then O^T += V^T P^T, one 32-key block at a time so that one block's softmax (vector ALU)
    // can overlap the other block's MFMAs. The reference max moves only when a block exceeds it
    // by more than kLazy (P <= 2^kLazy, harmless in float32 and bf16); O / l is exact for any
    // reference max, so the accumulator rescale is rare.
    const uint16_t* vsrc = sv + (((lane & 15) >> 2) + 4 * half) * VSTR + 16 * ((lane >> 4) & 1) +
                           4 * (lane & 3);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 pb[QB][2];
      bool rescale = false;
      float alpha[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qb][kb][r]);
        mx = xhalf_max(mx) * c;
        const bool up = mx > m_run[qb] + kLazy;
        const float m_new = up ? mx : m_run[qb];
        alpha[qb] = up ? fast_exp2(m_run[qb] - m_new) : 1.f;
        rescale = rescale || (up && m_run[qb] != kNegBig);  // O is still zero before any key
        m_run[qb] = m_new;
        float psum = 0.f;
        float pr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pr[r] = fast_exp2(fmaf(sacc[qb][kb][r], c, -m_new));
          psum += pr[r];
        }
#pragma unroll
        for (int st = 0; st < 2; ++st)
          pb[qb][st] = u32x4{pack_bf16(pr[8 * st + 0], pr[8 * st + 1]),
                             pack_bf16(pr[8 * st + 2], pr[8 * st + 3]),
                             pack_bf16(pr[8 * st + 4], pr[8 * st + 5]),
                             pack_bf16(pr[8 * st + 6], pr[8 * st + 7])};
        l_run[qb] = fmaf(l_run[qb], alpha[qb], psum);
      }
      if (__any(rescale)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha[qb];
      }
      // For d block db and key step st the A operand holds
      // V[key = kb*32 + 16 st + 8 (e / 4) + 4 half + e % 4][d = db*32 + lq], e = 0..7, fetched
      // with two transposing reads: this lane points at V[key0 + j][d0 + 4 q], j = (lane % 16)
      // / 4, q = lane % 4, where d0 = db*32 + 16 ((lane / 16) % 2) is its 16-lane group's first
      // dim.
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const uint16_t* pv = vsrc + (kb * 32 + 16 * st) * VSTR + db * 32;
          const u32x2 lo = ld_tr(pv);
          const u32x2 hi = ld_tr(pv + 8 * VSTR);
          const u32x4 va = u32x4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32(va, pb[qb][st], o[qb][db]);
        }
    }

  };

  for (int j = 0; j < ts.ntiles; j += 2) {
    if (j + 2 < ts.ntiles) load_tile(kb_, vb_, kbase, vbase, rs, ts.start(j + 2), S - 1);
    tile(j, 0);
    if (j + 1 < ts.ntiles) store_tile(ka_, va_, sK + K_TILE, sV + V_TILE);
    __syncthreads();
    if (j + 1 >= ts.ntiles) break;
    if (j + 3 < ts.ntiles) load_tile(ka_, va_, kbase, vbase, rs, ts.start(j + 3), S - 1);
    tile(j + 1, 1);
    if (j + 2 < ts.ntiles) store_tile(kb_, vb_, sK, sV);
    __syncthreads();
  }

  // normalise and write: lane holds query p, dims db*32 + 8 g + 4 half + (0..3)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = xhalf_sum(l_run[qb]);
    if (p[qb] < q1) {
      const int64_t row = (int64_t)(cu0 + p[qb]) * a.heads + h;
      store_row128<OUT>(reinterpret_cast<OUT*>(a.out) + row * kHeadDim, o[qb], 1.f / l_tot, half);
      // natural log-sum-exp of the scaled scores: m_run + log2(l) in the log2 domain, times ln 2
      if (a.lse != nullptr && half == 0)
        a.lse[row] = (m_run[qb] + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
    }
  }
}

}  // namespace

#ifndef RSWA_PREFILL_QB
#define RSWA_PREFILL_QB 1  // 32-query blocks per wave
#endif

hipError_t launch_prefill(const PrefillArgs& a, int out_f32, hipStream_t s) {
  constexpr int QB = RSWA_PREFILL_QB;
  constexpr int BMQ = kWavesPF * 32 * QB;
  const dim3 grid((a.max_seqlen + BMQ - 1) / BMQ, a.heads, a.nseq);
  if (out_f32)
    hipLaunchKernelGGL((prefill_kernel<float, QB>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_kernel<uint16_t, QB>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace rswa
