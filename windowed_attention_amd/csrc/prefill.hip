// K3: R-SWA-masked prefill / teacher-forced attention on bf16 MFMA (gfx950).
//
// Mask (deep dive "Unlimited-OCR", N(t) code block; GeekNews "Unlimited OCR", R-SWA section and the
// training section's packed multi-page sequences): in a sequence of S tokens whose first m are the
// reference prefix, query p sees
//   prefix key k < m: always (or only k <= p for prefix queries when the prefix is causal);
//   output key k >= m: iff k <= p and p - k < n (its own window of n outputs, itself included).
// A query tile therefore visits two key segments only: the prefix [0, m) and the window
// [max(m, q_first - n + 1), q_last]; every other key tile is skipped without being loaded. Element
// masks are applied only on blocks that need them (the prefix's ragged end, the causal-prefix
// diagonal, and the window), and the leading tiles that need none run a loop without mask tests.
//
// Tiling. A workgroup of 8 waves (512 threads, two waves per SIMD) owns 32 queries per wave of one
// (sequence, head); Q stays in registers for the whole key loop. Scores are formed transposed,
// S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the accumulator puts one query per lane (lane % 32)
// and 16 of a 32-key block's keys in that lane's registers, so the softmax max/sum over keys is
// in-lane plus one exchange with lane ^ 32. The output is also formed transposed, O^T = V^T P^T:
// the score registers, rounded to bf16, are already the B operand of the second MFMA (the key
// order inside a 16-key step is a permutation that the V^T operand follows), so P never leaves
// registers; the V^T operand comes out of gfx950's transposing LDS read.
//
// Key loop. K and V tiles of 64 keys are copied by LDS DMA (no register staging) into four
// XOR-swizzled buffers, three tiles ahead; one barrier per tile, in the middle of the tile's first
// step. The loop is software-pipelined over 32-key blocks: step b issues the score MFMAs of block
// b + 1 in between the vector-ALU softmax of block b, then the PV MFMAs of block b in between the
// rest of that softmax, and under its last MFMAs forms block b + 1's maximum and reads block
// b + 2's leading K fragments, so the matrix cores and the vector ALUs of a wave work at the same
// time. Softmax runs in the log2 domain in float32 with a lazily moved reference max; P is rounded
// to bf16 for the PV product and the output is normalised by the sum of P as rounded (so its
// weights sum to one). With a non-null lse the natural log-sum-exp of each query's scaled scores,
// from the float32 sum of the unrounded P, is written too (the training pass needs it).
#include "kernels.h"
#include "mfma.h"

namespace rswa {
namespace {

constexpr int kWavesPF = 8;               // waves per workgroup, 32 queries each
constexpr int kThreads = 64 * kWavesPF;
constexpr int BN = 64;                    // keys per tile
constexpr float kLazy = 8.f;              // log2-domain slack before the reference max moves

struct TileSched {
  int n_pre;   // tiles over the prefix segment [0, pre_end)
  int pre_end;
  int ws;      // first key of the window segment
  int ntiles;
  __device__ __forceinline__ int start(int j) const { return j < n_pre ? j * BN : ws + (j - n_pre) * BN; }
};

constexpr int T_TILE = BN * kHeadDim;               // swizzled K or V tile (bf16 elements)
constexpr int kDmaGroups = BN / 4 / kWavesPF;       // 4-row (1 KB) groups per wave per tile
constexpr int kDmaPieces = 2 * kDmaGroups;          // 16-byte DMA loads per wave per tile

// Tile k0 .. k0 + 63 of K and V (rows clamped to kmax) copied by LDS DMA into one buffer pair,
// swizzled: lane l of a 4-row group fetches the global chunk that belongs in LDS slot l % 16 of
// its row. With WIDE false the row offset is a 24-bit multiply (full rate; the launcher
// guarantees key * row_stride < 2^31, and at most 1024 heads keep row_stride below 2^24),
// instead of the quarter-rate 64-bit one.
template <bool WIDE>
__device__ __forceinline__ void dma_kv_tile(uint16_t* sk, uint16_t* sv, const uint16_t* kbase,
                                            const uint16_t* vbase, int row_stride, int k0,
                                            int kmax, int wave, int lane) {
#pragma unroll
  for (int u = 0; u < kDmaGroups; ++u) {
    const int grp = wave * kDmaGroups + u;
    const int row = 4 * grp + (lane >> 4);
    const int key = min(k0 + row, kmax);
    const int64_t roff = WIDE ? (int64_t)key * row_stride : (int64_t)__umul24(key, row_stride);
    const int64_t off = roff + 8 * ((lane & 15) ^ swz(row));  // this lane's LDS slot's chunk
    dma16(kbase + off, sk + grp * 4 * kHeadDim);
    dma16(vbase + off, sv + grp * 4 * kHeadDim);
  }
}

// A tile whose 64 rows all lie in [0, kmax]: no clamp, so the lanes' byte offsets within the tile
// (`voff`, computed once per kernel) are fixed and only the tile's wave-uniform base moves.
// `lk` / `lv`: LDS byte addresses of this wave's first group in the destination buffers.
__device__ __forceinline__ void dma_kv_tile_u(uint32_t lk, uint32_t lv, const uint16_t* kt,
                                              const uint16_t* vt, const uint32_t (&voff)[kDmaGroups]) {
#pragma unroll
  for (int u = 0; u < kDmaGroups; ++u) {
    dma16s(kt, voff[u], lk + u * 4 * kHeadDim * 2);
    dma16s(vt, voff[u], lv + u * 4 * kHeadDim * 2);
  }
}

// Scheduling fence: the interleave of MFMAs and vector-ALU work stays as written.
#define FENCE() __builtin_amdgcn_sched_barrier(0)

// The copy of tile j + 3 is issued at the middle of tile j, after the barrier that retires tile
// j - 1's buffer, and waited for two tiles later.
// LSE: also keep the float32 sum of the unrounded probabilities and write the log-sum-exp.
template <typename OUT, bool WIDE, bool LSE>
__global__ __launch_bounds__(kThreads, 8 / kWavesPF) void prefill_kernel(PrefillArgs a) {
  constexpr int BMQ = kWavesPF * 32;  // queries per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t sK[4 * T_TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[4 * T_TILE];

  // XCD-aware tile order: workgroups are dispatched round-robin over the 8 XCDs (workgroup i on
  // XCD i % 8), so giving each XCD a contiguous run of (query tile, head) pairs keeps one head's
  // query tiles together and its K / V tiles shared in that XCD's L2.
  int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
  {
    const int nx = gridDim.x, ny = gridDim.y, nwg = nx * ny * gridDim.z;
    if (nwg % 8 == 0) {
      const int i = bx + nx * (by + ny * bz);
      const int l = (i % 8) * (nwg / 8) + i / 8;
      bx = l % nx;
      by = (l / nx) % ny;
      bz = l / (nx * ny);
    }
  }
  const int s = bz, h = by;
  const int cu0 = a.cu_seqlens[s];
  const int S = a.cu_seqlens[s + 1] - cu0;
  // Metadata the host cannot see, checked once per (sequence, head) by the last tile of the grid:
  // a sequence longer than the grid covers (its rows past max_seqlen stay unwritten), a prefix
  // longer than its sequence or a window below 1 set the error word that rswa_prefill_check reads.
  if (bx == (int)gridDim.x - 1 && threadIdx.x == 0) {
    const int mm = a.prefix_len[s], nn = a.window[s];
    if (S < 0 || S > (int)gridDim.x * BMQ || mm < 0 || mm > S || nn < 1) *a.err = 1;
  }
  const int q0 = bx * BMQ;
  if (q0 >= S) return;
  const int q1 = min(q0 + BMQ, S);
  const int m = a.prefix_len[s];
  const int n = a.window[s];
  const bool pc = a.prefix_causal != 0;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, half = lane >> 5;
  const int64_t rs = (int64_t)a.heads * kHeadDim;
  const int64_t hoff = ((int64_t)cu0 * a.heads + h) * kHeadDim;
  const uint16_t* kbase = a.k + hoff;
  const uint16_t* vbase = a.v + hoff;
  // last key row a copy may touch; capped by max_seqlen so that the 24-bit offsets stay exact
  // even for a launch whose max_seqlen understates a sequence (its output is then incomplete)
  const int kmax = (WIDE ? S : min(S, a.max_seqlen)) - 1;

  const int p = q0 + wave * 32 + lq;
  u32x4 qf[8];
  {
    const int pq = min(p, S - 1);
#pragma unroll
    for (int st = 0; st < 8; ++st)
      qf[st] = *reinterpret_cast<const u32x4*>(a.q + hoff + pq * rs + st * 16 + half * 8);
  }
  // Materialise Q here: the compiler then waits for these loads once, before the loop, instead
  // of inside it, where its wait would also cover the tile copies in flight.
#pragma unroll
  for (int st = 0; st < 8; ++st) asm volatile("" : "+v"(qf[st]));

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
  const int nt = ts.ntiles;

  const int pre_hi = (pc && p < m) ? min(p, m - 1) : m - 1;
  const int win_lo = p >= m ? max(m, p - n + 1) : p + 1;

  const float c = a.scale_log2;
  // running reference max (log2 domain), the threshold past which it moves, the row sum of the
  // bf16-rounded probabilities (the output's normaliser) and, for the log-sum-exp, of the unrounded
  float m_run = kNegBig, m_thr = kNegBig, l_run = 0.f, l_exact = 0.f;
  floatx16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) zero16(o[db]);
  const SwzLane sl_(lane);
  const bf16x2v_t ones2 = {(__bf16)1.f, (__bf16)1.f};

  // scaled maximum of a score block over its 32 keys (16 in-lane, 16 in lane ^ 32)
  auto block_max = [&](const floatx16& x) {
    float mx = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
    return xhalf_max(mx) * c;
  };

  // element mask of the 32-key block kb of tile j, where that block is not fully visible;
  // returns whether it masked anything
  auto mask_block = [&](floatx16& sc, int j, int kb) {
    const int k0 = ts.start(j) + kb * 32;
    const bool is_pre = j < ts.n_pre;
    const bool need = is_pre ? (k0 + 32 > m || (pc && q0 < m && k0 + 31 > q0)) : true;
    if (need) {
      const int lo = is_pre ? 0 : win_lo;
      const int hi = is_pre ? pre_hi : p;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int k = k0 + 8 * (r >> 2) + 4 * half + (r & 3);
        sc[r] = (k >= lo && k <= hi) ? sc[r] : -INFINITY;
      }
    }
    return need;
  };

  // Row sum of the bf16-rounded probabilities that enter the PV product (two per dot2), so the
  // output's weights sum to one as rounded.
  auto rowsum8 = [&](const u32x4& pb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // copied out word by word: a bit_cast of the vector element compiles to the wrong register
      const uint32_t w = pb[i];
      bf16x2v_t pw;
      __builtin_memcpy(&pw, &w, sizeof(w));
      l_run = __builtin_amdgcn_fdot2_f32_bf16(pw, ones2, l_run, false);
    }
  };

  // One pipeline step: the softmax of block `cur` (scores complete, masked; `mxs` its scaled
  // maximum) under the score MFMAs of the next block (rows r_next of tile sk_next) into `nxt`,
  // then O^T += V^T P^T for `cur` (rows r_cur of tile sv_cur) under the rest of the softmax. The
  // maximum of `nxt` (before any mask) is formed under the last PV MFMAs and returned in `mxs`, so
  // that the next step starts with MFMAs rather than with a chain of vector-ALU maxima.
  // `kf` arrives holding the first four K fragments of the next block (read by the previous step)
  // and leaves holding those of the block after it (rows r_after of tile sk_after), read under the
  // last PV MFMAs into the registers the V operands free. `mid` runs between the two halves: the
  // tile barrier and the copy of a later tile, when this step has them.
  auto step = [&](floatx16& cur, floatx16& nxt, u32x4 (&kf)[4], const uint16_t* sk_next,
                  int r_next, const uint16_t* sv_cur, int r_cur, float& mxs, auto&& mid,
                  const uint16_t* sk_after, int r_after) {
    float m_new = 0.f;
    uint64_t up_mask = 0;  // lanes whose reference max moves (a scalar ballot)
    float pr[16];
    u32x4 va[4];
    FENCE();
    // While its score MFMAs and softmax interleave, a wave issues ahead of the other wave on its
    // SIMD (in this step layout equal priorities measure the same, within 0.3 %).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      nxt = mfma32(kf[i & 3], qf[i], i == 0 ? floatx16{} : nxt);
      if (i < 4) kf[i] = swz_ld_a(sk_next, sl_, r_next, i + 4);
      if (i >= 4) va[i - 4] = swz_ld_tr(sv_cur, sl_, r_cur, i - 4);
      if (i == 0) {
        // the reference max moves only when the block max passes it by kLazy
        const bool up = mxs > m_thr;
        up_mask = __builtin_amdgcn_ballot_w64(up);
        m_new = up ? mxs : m_run;
      } else {
        const int r = i - 1;  // exponentials 0..6 here, 7 below
        pr[r] = fast_exp2(fmaf(cur[r], c, -m_new));
      }
      FENCE();
    }
    pr[7] = fast_exp2(fmaf(cur[7], c, -m_new));
    u32x4 pb0 = u32x4{pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3]), pack_bf16(pr[4], pr[5]),
                      pack_bf16(pr[6], pr[7])};
    // computed here, under the score MFMAs, not sunk past the rescale branch to its use
    asm volatile("" : "+v"(pb0));
    FENCE();
    __builtin_amdgcn_s_setprio(0);
    mid();
    // Rare: some lane's reference max moved. Its accumulators and row sum are rescaled (lanes whose
    // max stayed get exp2(0) = 1; the first block of a row scales zeros).
    if (__builtin_expect(up_mask != 0, 0)) {
      const float alpha = fast_exp2(m_run - m_new);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      l_run *= alpha;
      if (LSE) l_exact *= alpha;
      m_run = m_new;
      m_thr = m_new + kLazy;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      o[db] = mfma32(va[db], pb0, o[db]);
      va[db] = swz_ld_tr(sv_cur, sl_, r_cur + 16, db);
      pr[8 + 2 * db] = fast_exp2(fmaf(cur[8 + 2 * db], c, -m_new));
      pr[9 + 2 * db] = fast_exp2(fmaf(cur[9 + 2 * db], c, -m_new));
      FENCE();
    }
    const u32x4 pb1 = u32x4{pack_bf16(pr[8], pr[9]), pack_bf16(pr[10], pr[11]),
                            pack_bf16(pr[12], pr[13]), pack_bf16(pr[14], pr[15])};
    rowsum8(pb0);
    float mn = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      o[db] = mfma32(va[db], pb1, o[db]);
      kf[db] = swz_ld_a(sk_after, sl_, r_after, db);
      if (db == 0) rowsum8(pb1);
      if (db == 1) {
        mn = fmaxf(nxt[0], nxt[1]);
#pragma unroll
        for (int r = 2; r < 8; ++r) mn = fmaxf(mn, nxt[r]);
      }
      if (db == 2) {
#pragma unroll
        for (int r = 8; r < 16; ++r) mn = fmaxf(mn, nxt[r]);
      }
      if (db == 3) mxs = xhalf_max(mn) * c;
      if (LSE) l_exact += (pr[4 * db] + pr[4 * db + 1]) + (pr[4 * db + 2] + pr[4 * db + 3]);
      FENCE();
    }
  };

  const int rs32 = (int)rs;
  // this lane's byte offsets within a tile, for the unclamped copies
  uint32_t voff[kDmaGroups];
#pragma unroll
  for (int u = 0; u < kDmaGroups; ++u) {
    const int row = 4 * (wave * kDmaGroups + u) + (lane >> 4);
    voff[u] = 2u * (uint32_t)(row * rs32 + 8 * ((lane & 15) ^ swz(row)));
  }
  // LDS byte addresses of this wave's first DMA group in buffer 0 (taken once: the generic to LDS
  // conversion carries a null test)
  const uint32_t lk0 = lds_addr(sK + wave * kDmaGroups * 4 * kHeadDim);
  const uint32_t lv0 = lds_addr(sV + wave * kDmaGroups * 4 * kHeadDim);
  // copy of an unclamped tile (first key k0, k0 + BN - 1 <= kmax) into buffer b
  auto issue_u = [&](int k0, int b) {
    // byte offset of the tile: a 32-bit product when the narrow-offset bound holds
    const uint16_t* kt;
    const uint16_t* vt;
    if (WIDE) {
      kt = kbase + (int64_t)k0 * rs;
      vt = vbase + (int64_t)k0 * rs;
    } else {
      const uint32_t tb = 2u * (uint32_t)k0 * (uint32_t)rs32;
      kt = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(kbase) + tb);
      vt = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(vbase) + tb);
    }
    dma_kv_tile_u(lk0 + b * T_TILE * 2, lv0 + b * T_TILE * 2, kt, vt, voff);
  };
  // copy tile j into buffer b (= j % 4)
  auto issue_to = [&](int j, int b) {
    const int k0 = ts.start(j);
    if (__builtin_expect(k0 + BN - 1 <= kmax, 1))
      issue_u(k0, b);
    else
      dma_kv_tile<WIDE>(sK + b * T_TILE, sV + b * T_TILE, kbase, vbase, rs32, k0, kmax, wave,
                        lane);
  };
  auto issue = [&](int j) { issue_to(j, j & 3); };
  issue(0);
  if (nt > 1) issue(1);
  if (nt > 2) issue(2);
  if (nt > 2)
    dma_wait_barrier<2 * kDmaPieces>();
  else if (nt > 1)
    dma_wait_barrier<kDmaPieces>();
  else
    dma_wait_barrier<0>();

  floatx16 s0, s1;
  zero16(s0);
#pragma unroll
  for (int st = 0; st < 8; ++st) s0 = mfma32(swz_ld_a(sK, sl_, 0, st), qf[st], s0);
  mask_block(s0, 0, 0);
  float mxs = block_max(s0);
  u32x4 kf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kf[i] = swz_ld_a(sK, sl_, 32, i);
  auto none = [] {};

  // Leading tiles that need no element mask (inside the prefix, and below the diagonal of a
  // causal prefix) run a loop without mask tests or end-of-loop cases.
  int n_plain = min(m / BN, ts.n_pre);
  if (pc && q0 < m) n_plain = min(n_plain, (q0 + 1) / BN);
  const int j_plain = min(n_plain - 1, nt - 3);
  // leading prefix tiles whose copies need no clamp
  const int n_fast = min(ts.n_pre, (kmax + 1) / BN);
  int j = 0;
  // four tiles per iteration, so that every LDS buffer offset is a constant; the tiles it copies
  // (j + 3 .. j + 6) are unclamped prefix tiles
  for (; j + 4 <= j_plain && j + 7 <= n_fast; j += 4) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint16_t* k_j = sK + b * T_TILE;
      const uint16_t* v_j = sV + b * T_TILE;
      const uint16_t* k_n = sK + ((b + 1) & 3) * T_TILE;
      step(s0, s1, kf, k_j, 32, v_j, 0, mxs, [&] {
        dma_wait_barrier<kDmaPieces>();
        issue_u((j + b + 3) * BN, (b + 3) & 3);
      }, k_n, 0);
      step(s1, s0, kf, k_n, 0, v_j, 32, mxs, none, k_n, 32);
    }
  }
  for (; j < j_plain; ++j) {
    const uint16_t* k_j = sK + (j & 3) * T_TILE;
    const uint16_t* v_j = sV + (j & 3) * T_TILE;
    const uint16_t* k_n = sK + ((j + 1) & 3) * T_TILE;
    step(s0, s1, kf, k_j, 32, v_j, 0, mxs, [&] {
      dma_wait_barrier<kDmaPieces>();
      issue(j + 3);
    }, k_n, 0);
    step(s1, s0, kf, k_n, 0, v_j, 32, mxs, none, k_n, 32);
  }
  for (; j < nt; ++j) {
    const uint16_t* k_j = sK + (j & 3) * T_TILE;
    const uint16_t* v_j = sV + (j & 3) * T_TILE;
    const uint16_t* k_n = sK + ((j + 1) & 3) * T_TILE;
    // tile j + 1 must have landed (tile j + 2's copy may still be in flight); past this barrier
    // every wave is done with tile j - 1, whose buffer takes tile j + 3
    step(s0, s1, kf, k_j, 32, v_j, 0, mxs, [&] {
      if (j + 2 < nt)
        dma_wait_barrier<kDmaPieces>();
      else
        dma_wait_barrier<0>();
      if (j + 3 < nt) issue(j + 3);
    }, k_n, 0);
    if (mask_block(s1, j, 1)) mxs = block_max(s1);
    step(s1, s0, kf, k_n, 0, v_j, 32, mxs, none, k_n, 32);
    if (j + 1 < nt && mask_block(s0, j + 1, 0)) mxs = block_max(s0);
  }

  const float l_tot = xhalf_sum(l_run);
  if (p < q1) {
    const int64_t row = (int64_t)(cu0 + p) * a.heads + h;
    store_row128<OUT>(reinterpret_cast<OUT*>(a.out) + row * kHeadDim, o, 1.f / l_tot, half);
    if (LSE) {
      const float le = xhalf_sum(l_exact);
      if (half == 0) a.lse[row] = (m_run + __builtin_amdgcn_logf(le)) * 0.69314718055994531f;
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int out_f32, hipStream_t s) {
  constexpr int BMQ = kWavesPF * 32;
  const dim3 grid((a.max_seqlen + BMQ - 1) / BMQ, a.heads, a.nseq);
  // 24-bit row offsets hold when (max_seqlen - 1) * heads * 128 < 2^31
  const bool wide = (int64_t)a.max_seqlen * a.heads * kHeadDim >= (int64_t{1} << 31);
  const bool lse = a.lse != nullptr;
#define RSWA_PREFILL_LAUNCH(OUT, W, L) \
  hipLaunchKernelGGL((prefill_kernel<OUT, W, L>), grid, dim3(kThreads), 0, s, a)
  if (lse) {
    if (out_f32 && wide) RSWA_PREFILL_LAUNCH(float, true, true);
    else if (out_f32) RSWA_PREFILL_LAUNCH(float, false, true);
    else if (wide) RSWA_PREFILL_LAUNCH(uint16_t, true, true);
    else RSWA_PREFILL_LAUNCH(uint16_t, false, true);
  } else {
    if (out_f32 && wide) RSWA_PREFILL_LAUNCH(float, true, false);
    else if (out_f32) RSWA_PREFILL_LAUNCH(float, false, false);
    else if (wide) RSWA_PREFILL_LAUNCH(uint16_t, true, false);
    else RSWA_PREFILL_LAUNCH(uint16_t, false, false);
  }
#undef RSWA_PREFILL_LAUNCH
  return hipGetLastError();
}

}  // namespace rswa
