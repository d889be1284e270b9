// Backward of the R-SWA-masked teacher-forced attention (dQ, dK, dV) on bf16 MFMA (gfx950).
//
// The pages train the decoder on packed 32K-token sequences of prefix + output documents
// (GeekNews "Unlimited OCR", training section; deep dive "Unlimited-OCR", training setup table);
// the mask is the prefill's (deep dive, N(t) code block): query p sees every prefix key (only
// k <= p for prefix queries when the prefix is causal) and the outputs k in (p - n, p]. With
// P = softmax(scale Q K^T) under that mask, O = P V and the incoming gradient dO:
//   delta_p = sum_d dO[p][d] O[p][d]          (= sum_k P[p][k] dP[p][k])
//   dP = dO V^T,  dS = P * (dP - delta),  dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
// P is recomputed from the forward's log-sum-exp: P[p][k] = 2^(s c - lse_p log2 e), c = scale
// log2 e, so no softmax state is kept between the passes.
//
// Three kernels, no atomics and no partial sums:
//   delta: one 16-lane group per (token, head) row, HBM-bound.
//   dK/dV: key-parallel. A workgroup owns 32 keys per wave; the wave keeps K and V of its keys in
//     registers (B operands) and its dK^T, dV^T accumulators in registers, and streams the query
//     tiles that can see its keys (every query for a prefix key, the n queries of the window for
//     an output key) through LDS: Q and dO tiles row-major, read both straight (S = Q K^T,
//     dP = dO V^T) and through the transposing LDS read (dV^T = dO^T P, dK^T = Q^T dS).
//   dQ: query-parallel, the forward's tiling: Q and dO of 32 queries per wave in registers, K and
//     V tiles of the prefix segment and the window segment through LDS, S^T = K Q^T,
//     dP^T = V dO^T, dQ^T = K^T dS^T (K^T from the transposing read).
// P and dS are rounded to bf16 for the MFMA products; every sum runs in float32.
#include "kernels.h"
#include "mfma.h"

namespace rswa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------------------------------
// delta_p = rowsum(dO * O) per (token, head) row: 16 lanes x 8 dims per row
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8]) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = a[i];
    x[2 * i] = bf16_lo(w);
    x[2 * i + 1] = bf16_hi(w);
  }
}

template <typename OT>
__global__ __launch_bounds__(256) void delta_kernel(const OT* __restrict__ out,
                                                    const uint16_t* __restrict__ dout,
                                                    float* __restrict__ delta, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  const int64_t rr = row < rows ? row : rows - 1;
  float o[8], g[8];
  load8(out + rr * kHeadDim + c * 8, o);
  load8(dout + rr * kHeadDim + c * 8, g);
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = fmaf(o[i], g[i], acc);
  acc = row16_sum(acc);
  if (c == 0 && row < rows) delta[row] = acc;
}

// ------------------------------------------------------------------------------------------
// dK / dV: key-parallel
// ------------------------------------------------------------------------------------------
#ifndef RSWA_KV_WAVES
#define RSWA_KV_WAVES 4  // waves per workgroup, 32 keys each
#endif
#ifndef RSWA_KV_QPAD
#define RSWA_KV_QPAD 8   // bf16 pad per Q / dO tile row
#endif
constexpr int kKvWaves = RSWA_KV_WAVES;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int BNK = 32 * kKvWaves;                 // keys per workgroup
constexpr int BMQ = 64;                            // queries per LDS tile
constexpr int QSTR = kHeadDim + RSWA_KV_QPAD;      // Q / dO tile row stride (bf16)
constexpr int Q_TILE = BMQ * QSTR;
constexpr int kRowsPerThread = BMQ * 16 / kKvThreads;  // 16-byte pieces per thread per tensor

struct QTileRegs {
  u32x4 q[kRowsPerThread];
  u32x4 g[kRowsPerThread];
  float aux;  // lse (threads < BMQ) or delta (threads BMQ .. 2 BMQ - 1)
};

__device__ __forceinline__ void load_qtile(QTileRegs& r, const uint16_t* qbase,
                                           const uint16_t* gbase, const float* lse,
                                           const float* delta, int64_t rs, int heads, int p0,
                                           int pmax) {
  const int t = threadIdx.x;
  const int c = t & 15, rg = t >> 4;
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const int p = min(p0 + rg * kRowsPerThread + u, pmax);
    r.q[u] = *reinterpret_cast<const u32x4*>(qbase + p * rs + c * 8);
    r.g[u] = *reinterpret_cast<const u32x4*>(gbase + p * rs + c * 8);
  }
  if (t < 2 * BMQ) {
    const int p = min(p0 + (t & (BMQ - 1)), pmax);
    r.aux = t < BMQ ? lse[(int64_t)p * heads] * kLog2e : delta[(int64_t)p * heads];
  }
}

__device__ __forceinline__ void store_qtile(const QTileRegs& r, uint16_t* sq, uint16_t* sg,
                                            float* sl, float* sd) {
  const int t = threadIdx.x;
  const int c = t & 15, rg = t >> 4;
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    *reinterpret_cast<u32x4*>(sq + (rg * kRowsPerThread + u) * QSTR + c * 8) = r.q[u];
    *reinterpret_cast<u32x4*>(sg + (rg * kRowsPerThread + u) * QSTR + c * 8) = r.g[u];
  }
  if (t < BMQ) sl[t] = r.aux;
  else if (t < 2 * BMQ) sd[t - BMQ] = r.aux;
}

template <typename OUT>
__global__ __launch_bounds__(kKvThreads) void dkdv_kernel(BwdArgs a, int nkb) {
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2 * Q_TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sG[2 * Q_TILE];
  __shared__ __attribute__((aligned(16))) float sL[2 * BMQ];
  __shared__ __attribute__((aligned(16))) float sD[2 * BMQ];

  // key blocks outermost across heads: the prefix blocks (long query loops) start first
  const int idx = blockIdx.x;
  const int h = idx % a.heads;
  const int kblk = (idx / a.heads) % nkb;
  const int s = idx / (a.heads * nkb);
  const int cu0 = a.cu_seqlens[s];
  const int S = a.cu_seqlens[s + 1] - cu0;
  const int k0 = kblk * BNK;
  if (k0 >= S) return;
  const int m = a.prefix_len[s];
  const int n = a.window[s];
  const bool pc = a.prefix_causal != 0;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, half = lane >> 5;
  const int64_t rs = (int64_t)a.heads * kHeadDim;
  const int64_t hoff = ((int64_t)cu0 * a.heads + h) * kHeadDim;
  const uint16_t* qbase = a.q + hoff;
  const uint16_t* gbase = a.dout + hoff;
  const float* lse = a.lse + (int64_t)cu0 * a.heads + h;
  const float* dlt = a.delta + (int64_t)cu0 * a.heads + h;

  // this lane's key and its K / V rows as B operands (8 d-steps of 16)
  const int wk0 = k0 + wave * 32;
  const int kw = wk0 + lq;
  u32x4 kf[8], vf[8];
  {
    const int kc = min(kw, S - 1);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      kf[st] = *reinterpret_cast<const u32x4*>(a.k + hoff + kc * rs + st * 16 + half * 8);
      vf[st] = *reinterpret_cast<const u32x4*>(a.v + hoff + kc * rs + st * 16 + half * 8);
    }
  }
  // queries that see key kw: [plo, phi)
  int plo, phi;
  if (kw >= S) {
    plo = phi = 0;
  } else if (kw < m) {
    plo = pc ? kw : 0;
    phi = S;
  } else {
    plo = kw;
    phi = min(S, kw + n);
  }
  // ... and the union over this wave's keys, and over the workgroup's
  int wq_lo = 0, wq_hi = 0;
  if (wk0 < S) {
    const int wlast = min(wk0 + 31, S - 1);
    wq_lo = wk0 < m ? (pc ? wk0 : 0) : wk0;
    wq_hi = wk0 < m ? S : min(S, wlast + n);
  }
  const int klast = min(k0 + BNK, S) - 1;
  const int qlo = k0 < m ? (pc ? k0 : 0) : k0;
  const int qhi = k0 < m ? S : min(S, klast + n);
  const int ntiles = (qhi - qlo + BMQ - 1) / BMQ;
  // every (query, key) pair of a tile is visible when all the wave's keys are prefix keys and,
  // with a causal prefix, the tile's first query is at or after the wave's last key
  const bool wave_pre = wk0 + 32 <= min(m, S);

  const float c = a.scale_log2;
  floatx16 dk[4], dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    zero16(dk[db]);
    zero16(dv[db]);
  }

  const uint16_t* qtr = tr_base(sQ, QSTR, lane);
  const uint16_t* gtr = tr_base(sG, QSTR, lane);

  QTileRegs regs;
  load_qtile(regs, qbase, gbase, lse, dlt, rs, a.heads, qlo, S - 1);
  store_qtile(regs, sQ, sG, sL, sD);
  if (ntiles > 1) load_qtile(regs, qbase, gbase, lse, dlt, rs, a.heads, qlo + BMQ, S - 1);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    const int qt0 = qlo + j * BMQ;
    const uint16_t* sq = sQ + buf * Q_TILE;
    const uint16_t* sg = sG + buf * Q_TILE;
    const float* sl = sL + buf * BMQ;
    const float* sd = sD + buf * BMQ;
    const bool full = wave_pre && qt0 + BMQ <= S && (!pc || qt0 >= wk0 + 31);
#pragma unroll
    for (int qb = 0; qb < BMQ / 32; ++qb) {
      const int pb0 = qt0 + qb * 32;
      if (pb0 >= wq_hi || pb0 + 32 <= wq_lo) continue;  // wave-uniform
      floatx16 sacc, dpacc;
      zero16(sacc);
      zero16(dpacc);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const u32x4 qa =
            *reinterpret_cast<const u32x4*>(sq + (qb * 32 + lq) * QSTR + st * 16 + half * 8);
        sacc = mfma32(qa, kf[st], sacc);
      }
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const u32x4 ga =
            *reinterpret_cast<const u32x4*>(sg + (qb * 32 + lq) * QSTR + st * 16 + half * 8);
        dpacc = mfma32(ga, vf[st], dpacc);
      }
      // accumulator register r: query pb0 + 8 (r / 4) + 4 half + r % 4, key kw
      float pr[16], ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 l4 = *reinterpret_cast<const float4*>(sl + qb * 32 + 8 * g + 4 * half);
        const float4 d4 = *reinterpret_cast<const float4*>(sd + qb * 32 + 8 * g + 4 * half);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g + i;
          float x = fast_exp2(fmaf(sacc[r], c, -lv[i]));
          if (!full) {
            const int p = pb0 + 8 * g + 4 * half + i;
            x = (p >= plo && p < phi) ? x : 0.f;
          }
          pr[r] = x;
          ds[r] = x * (dpacc[r] - dv4[i]);
        }
      }
      const u32x4 pb[2] = {pack_b(pr, 0), pack_b(pr, 1)};
      const u32x4 sb[2] = {pack_b(ds, 0), pack_b(ds, 1)};
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const u32x4 ga = ld_tr_op(gtr + buf * Q_TILE, QSTR, qb * 32 + 16 * st, db * 32);
          dv[db] = mfma32(ga, pb[st], dv[db]);
        }
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const u32x4 qa = ld_tr_op(qtr + buf * Q_TILE, QSTR, qb * 32 + 16 * st, db * 32);
          dk[db] = mfma32(qa, sb[st], dk[db]);
        }
    }
    if (j + 1 < ntiles)
      store_qtile(regs, sQ + (buf ^ 1) * Q_TILE, sG + (buf ^ 1) * Q_TILE, sL + (buf ^ 1) * BMQ,
                  sD + (buf ^ 1) * BMQ);
    if (j + 2 < ntiles)
      load_qtile(regs, qbase, gbase, lse, dlt, rs, a.heads, qlo + (j + 2) * BMQ, S - 1);
    __syncthreads();
  }

  if (kw < S) {
    const int64_t row = ((int64_t)(cu0 + kw) * a.heads + h) * kHeadDim;
    store_row128<OUT>(reinterpret_cast<OUT*>(a.dk) + row, dk, a.scale, half);
    store_row128<OUT>(reinterpret_cast<OUT*>(a.dv) + row, dv, 1.f, half);
  }
}

// ------------------------------------------------------------------------------------------
// dQ: query-parallel (the forward's key schedule)
// ------------------------------------------------------------------------------------------
#ifndef RSWA_DQ_WAVES
#define RSWA_DQ_WAVES 8  // waves per workgroup, 32 queries each
#endif
#ifndef RSWA_DQ_KPAD
#define RSWA_DQ_KPAD 8   // bf16 pad per K / V tile row
#endif
constexpr int kDqWaves = RSWA_DQ_WAVES;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int BNQ = 32 * kDqWaves;                  // queries per workgroup
constexpr int BN = 64;                              // keys per tile
constexpr int KSTR = kHeadDim + RSWA_DQ_KPAD;
constexpr int K_TILE = BN * KSTR;
constexpr int kKeyPieces = BN * 16 / kDqThreads;    // 16-byte pieces per thread per tensor

struct KTileRegs {
  u32x4 k[kKeyPieces];
  u32x4 v[kKeyPieces];
};

__device__ __forceinline__ void load_ktile(KTileRegs& r, const uint16_t* kbase,
                                           const uint16_t* vbase, int64_t rs, int k0, int kmax) {
  const int t = threadIdx.x;
  const int c = t & 15, kg = t >> 4;
#pragma unroll
  for (int u = 0; u < kKeyPieces; ++u) {
    const int key = min(k0 + kg * kKeyPieces + u, kmax);
    r.k[u] = *reinterpret_cast<const u32x4*>(kbase + key * rs + c * 8);
    r.v[u] = *reinterpret_cast<const u32x4*>(vbase + key * rs + c * 8);
  }
}

__device__ __forceinline__ void store_ktile(const KTileRegs& r, uint16_t* sk, uint16_t* sv) {
  const int t = threadIdx.x;
  const int c = t & 15, kg = t >> 4;
#pragma unroll
  for (int u = 0; u < kKeyPieces; ++u) {
    *reinterpret_cast<u32x4*>(sk + (kg * kKeyPieces + u) * KSTR + c * 8) = r.k[u];
    *reinterpret_cast<u32x4*>(sv + (kg * kKeyPieces + u) * KSTR + c * 8) = r.v[u];
  }
}

template <typename OUT>
__global__ __launch_bounds__(kDqThreads) void dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2 * K_TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2 * K_TILE];

  const int s = blockIdx.z, h = blockIdx.y;
  const int cu0 = a.cu_seqlens[s];
  const int S = a.cu_seqlens[s + 1] - cu0;
  const int q0 = blockIdx.x * BNQ;
  if (q0 >= S) return;
  const int q1 = min(q0 + BNQ, S);
  const int m = a.prefix_len[s];
  const int n = a.window[s];
  const bool pc = a.prefix_causal != 0;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, half = lane >> 5;
  const int64_t rs = (int64_t)a.heads * kHeadDim;
  const int64_t hoff = ((int64_t)cu0 * a.heads + h) * kHeadDim;
  const uint16_t* kbase = a.k + hoff;
  const uint16_t* vbase = a.v + hoff;

  // this lane's query, its Q and dO rows as B operands, its lse (log2 domain) and delta
  const int p = q0 + wave * 32 + lq;
  const int pq = min(p, S - 1);
  u32x4 qf[8], gf[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    qf[st] = *reinterpret_cast<const u32x4*>(a.q + hoff + pq * rs + st * 16 + half * 8);
    gf[st] = *reinterpret_cast<const u32x4*>(a.dout + hoff + pq * rs + st * 16 + half * 8);
  }
  const int64_t prow = (int64_t)(cu0 + pq) * a.heads + h;
  const float lse2 = a.lse[prow] * kLog2e;
  const float dlt = a.delta[prow];

  // key tiles: the prefix segment, then the output window segment (as in the forward)
  const int pre_end = (pc && q1 <= m) ? q1 : m;
  const int n_pre = (pre_end + BN - 1) / BN;
  int ws = 0, n_win = 0;
  if (q1 > m) {
    ws = max(m, max(q0, m) - n + 1);
    n_win = (q1 - ws + BN - 1) / BN;
  }
  const int ntiles = n_pre + n_win;
  auto tstart = [&](int j) { return j < n_pre ? j * BN : ws + (j - n_pre) * BN; };
  const int pre_hi = (pc && p < m) ? min(p, m - 1) : m - 1;
  const int win_lo = p >= m ? max(m, p - n + 1) : p + 1;

  const float c = a.scale_log2;
  floatx16 dq[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) zero16(dq[db]);
  const uint16_t* ktr = tr_base(sK, KSTR, lane);

  KTileRegs regs;
  load_ktile(regs, kbase, vbase, rs, tstart(0), S - 1);
  store_ktile(regs, sK, sV);
  if (ntiles > 1) load_ktile(regs, kbase, vbase, rs, tstart(1), S - 1);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    const uint16_t* sk = sK + buf * K_TILE;
    const uint16_t* sv = sV + buf * K_TILE;
    const int k0 = tstart(j);
    const bool is_pre = j < n_pre;
    const bool need_mask = is_pre ? (k0 + BN > m || (pc && q0 < m && k0 + BN - 1 > q0)) : true;
    const int lo = is_pre ? 0 : win_lo;
    const int hi = is_pre ? pre_hi : p;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      floatx16 sacc, dpacc;
      zero16(sacc);
      zero16(dpacc);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const u32x4 ka =
            *reinterpret_cast<const u32x4*>(sk + (kb * 32 + lq) * KSTR + st * 16 + half * 8);
        sacc = mfma32(ka, qf[st], sacc);
      }
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const u32x4 va =
            *reinterpret_cast<const u32x4*>(sv + (kb * 32 + lq) * KSTR + st * 16 + half * 8);
        dpacc = mfma32(va, gf[st], dpacc);
      }
      // accumulator register r: key k0 + kb*32 + 8 (r / 4) + 4 half + r % 4, query p
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = fast_exp2(fmaf(sacc[r], c, -lse2));
        if (need_mask) {
          const int k = k0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          x = (k >= lo && k <= hi) ? x : 0.f;
        }
        ds[r] = x * (dpacc[r] - dlt);
      }
      const u32x4 sb[2] = {pack_b(ds, 0), pack_b(ds, 1)};
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const u32x4 ka = ld_tr_op(ktr + buf * K_TILE, KSTR, kb * 32 + 16 * st, db * 32);
          dq[db] = mfma32(ka, sb[st], dq[db]);
        }
    }
    if (j + 1 < ntiles) store_ktile(regs, sK + (buf ^ 1) * K_TILE, sV + (buf ^ 1) * K_TILE);
    if (j + 2 < ntiles) load_ktile(regs, kbase, vbase, rs, tstart(j + 2), S - 1);
    __syncthreads();
  }

  if (p < q1)
    store_row128<OUT>(reinterpret_cast<OUT*>(a.dq) + ((int64_t)(cu0 + p) * a.heads + h) * kHeadDim,
                      dq, a.scale, half);
}

}  // namespace

hipError_t launch_prefill_bwd(const BwdArgs& a, int out_f32, int grad_f32, int64_t total,
                              hipStream_t s) {
  const int64_t rows = total * a.heads;
  if (rows > 0) {
    const dim3 g((unsigned)((rows + 15) / 16));
    if (out_f32)
      hipLaunchKernelGGL(delta_kernel<float>, g, dim3(256), 0, s,
                         reinterpret_cast<const float*>(a.out), a.dout, a.delta, rows);
    else
      hipLaunchKernelGGL(delta_kernel<uint16_t>, g, dim3(256), 0, s,
                         reinterpret_cast<const uint16_t*>(a.out), a.dout, a.delta, rows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nkb = (a.max_seqlen + BNK - 1) / BNK;
  const dim3 gkv((unsigned)nkb * a.heads * a.nseq);
  const dim3 gq((a.max_seqlen + BNQ - 1) / BNQ, a.heads, a.nseq);
  if (grad_f32) {
    hipLaunchKernelGGL(dkdv_kernel<float>, gkv, dim3(kKvThreads), 0, s, a, nkb);
    hipLaunchKernelGGL(dq_kernel<float>, gq, dim3(kDqThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(dkdv_kernel<uint16_t>, gkv, dim3(kKvThreads), 0, s, a, nkb);
    hipLaunchKernelGGL(dq_kernel<uint16_t>, gq, dim3(kDqThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace rswa
