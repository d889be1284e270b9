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
//   delta: one 16-lane group per (token, head) row, HBM-bound; it stores -delta and lse in the
//     log2 domain in the caller's work array.
//   dK/dV: key-parallel. A workgroup owns 32 keys per wave; the wave keeps K and V of its keys in
//     registers (B operands) and its dK^T, dV^T accumulators in registers, and streams the query
//     tiles that can see its keys (every query for a prefix key, the n queries of the window for
//     an output key) through LDS: Q and dO tiles row-major, read both straight (S = Q K^T,
//     dP = dO V^T) and through the transposing LDS read (dV^T = dO^T P, dK^T = Q^T dS). The
//     loop over 32-query blocks is software-pipelined: S and dP of the next block are issued
//     while P and dS of the current block are formed.
//   dQ: query-parallel, the forward's tiling: Q and dO of 32 queries per wave in registers, K and
//     V tiles of the prefix segment and the window segment through LDS, S^T = K Q^T,
//     dP^T = V dO^T, dQ^T = K^T dS^T (K^T from the transposing read).
// P and dS are rounded to bf16 for the MFMA products; every sum runs in float32.
#include "kernels.h"
#include "mfma.h"

namespace rswa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Scheduling fence: the interleave of MFMAs, LDS reads and vector-ALU work stays as written.
#define FENCE() __builtin_amdgcn_sched_barrier(0)

// v_mfma_f32_32x32x16_bf16 with its accumulator in VGPRs (the vector ALU reads S and dP) and its B
// operand in AGPRs. Written as inline assembly because the compiler gives every MFMA of a kernel
// that uses AGPRs an AGPR accumulator and then copies S and dP out register by register. The
// compiler does not see these as MFMAs, so the wait states their hazards need are provided here:
// a chain accumulates in place (same opcode, exact overlap: none needed); a start value written by
// the vector ALU gets two before the first MFMA reads it (mfma_vacc_first); gfx950 needs 12 wait
// states between an MFMA and any other instruction that reads or writes its result, which the
// 16 MFMAs of the step's other product half provide where the results stay in place, and
// mfma_vacc_last2 (the last MFMAs of the S and dP chains issued together, then 12 wait states)
// where the compiler moves them to other registers right away. LDS-loaded operands are covered
// by the compiler's lgkmcnt waits on the asm inputs. A test checks every distance on the
// compiled assembly.
__device__ __forceinline__ void mfma_vacc_zero(floatx16& d, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_vacc(floatx16& d, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_vacc_first(floatx16& d, const u32x4& a, const u32x4& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
struct Guarded { static constexpr bool value = true; };
struct Unguarded { static constexpr bool value = false; };
__device__ __forceinline__ void mfma_vacc_last2(floatx16& d0, const u32x4& a0, const u32x4& b0,
                                                floatx16& d1, const u32x4& a1, const u32x4& b1) {
  asm volatile(
      "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1\n\t"
      "s_nop 7\n\ts_nop 3"
      : "+v"(d0), "+v"(d1)
      : "v"(a0), "a"(b0), "v"(a1), "a"(b1));
}

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

// Also converts the forward's natural-log lse to the log2 domain the other kernels use. The work
// array is head-major, so that a tile of consecutive queries of one head reads its lse and delta
// from one contiguous run: work[0][h][token] = lse * log2(e), work[1][h][token] = -delta (the dP
// chains start from it). A workgroup takes 32 consecutive tokens of one head (two 16-token passes
// of its 16 lane groups), so its work values fill whole 128-byte lines; heads run fastest across
// workgroups, so the workgroups in flight read one contiguous run of O and dO rows.
template <typename OT>
__global__ __launch_bounds__(256) void delta_kernel(const OT* __restrict__ out,
                                                    const uint16_t* __restrict__ dout,
                                                    const float* __restrict__ lse,
                                                    float* __restrict__ work, int64_t total,
                                                    int heads) {
  const int h = (int)(blockIdx.x % (unsigned)heads);
  const int64_t t0 = (int64_t)(blockIdx.x / (unsigned)heads) * 32;
  const int64_t rows = total * heads;
  const int c = threadIdx.x & 15;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t t = t0 + 16 * u + (threadIdx.x >> 4);
    const int64_t row = (t < total ? t : total - 1) * heads + h;
    float o[8], g[8];
    load8(out + row * kHeadDim + c * 8, o);
    load8(dout + row * kHeadDim + c * 8, g);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(o[i], g[i], acc);
    acc = row16_sum(acc);
    if (t < total) {
      if (c == 0) work[rows + h * total + t] = -acc;
      if (c == 1) work[h * total + t] = lse[row] * kLog2e;
    }
  }
}

// ------------------------------------------------------------------------------------------
// dK / dV: key-parallel
// ------------------------------------------------------------------------------------------
#ifndef RSWA_KV_WAVES
#define RSWA_KV_WAVES 4  // waves per workgroup, 32 keys each
#endif
constexpr int kKvWaves = RSWA_KV_WAVES;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int BNK = 32 * kKvWaves;                 // keys per workgroup
constexpr int BMQ = 64;                            // queries per LDS tile
constexpr int Q_TILE = BMQ * kHeadDim;             // swizzled Q / dO tile (bf16 elements)

constexpr int kGroupsPerWave = BMQ / 4 / kKvWaves;   // 4-row (1 KB) groups per wave
constexpr int kKvPieces = 2 * kGroupsPerWave;         // 16-byte DMA loads per wave per tile

// Tile p0 .. p0 + 63 of Q and dO (rows clamped to pmax) and its lse / delta, copied by LDS DMA
// into one buffer set. The lse / delta loads go first: with the 16-byte pieces issued after them,
// "at most kKvPieces outstanding" then means every earlier tile has landed on every wave.
__device__ __forceinline__ void dma_qtile(uint16_t* sq, uint16_t* sg, float* sl, float* sd,
                                          const uint16_t* qbase, const uint16_t* gbase,
                                          const float* lse, const float* dlt, int64_t rs,
                                          int p0, int pmax, int wave, int lane) {
  if (wave == 0) dma4(lse + min(p0 + lane, pmax), sl);
  if (wave == 1) dma4(dlt + min(p0 + lane, pmax), sd);
#pragma unroll
  for (int u = 0; u < kGroupsPerWave; ++u) {
    const int grp = wave * kGroupsPerWave + u;
    const int row = 4 * grp + (lane >> 4);
    const int c = (lane & 15) ^ swz(row);  // this lane's LDS slot holds chunk c of its row
    const int64_t off = (int64_t)min(p0 + row, pmax) * rs + c * 8;
    dma16(qbase + off, sq + grp * 4 * kHeadDim);
    dma16(gbase + off, sg + grp * 4 * kHeadDim);
  }
}

// Each wave walks every 32-query block of the workgroup's query range (blocks its keys cannot see
// are masked out); step b issues S and dP of block b + 1 in between the vector-ALU work of block b
// (P, dS and their bf16 packing), then dV^T and dK^T of block b, so a wave's matrix cores are fed
// while its P / dS are formed. Four buffer sets: the copy of tile j + 3 goes out at the middle of
// tile j, after the barrier that retires tile j - 1's buffers.
template <typename OUT>
__global__ __launch_bounds__(kKvThreads) void dkdv_kernel(BwdArgs a, int nkb) {
  __shared__ __attribute__((aligned(16))) uint16_t sQ[4 * Q_TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sG[4 * Q_TILE];
  __shared__ __attribute__((aligned(16))) float sL[2 * kKvWaves * BMQ];
  __shared__ __attribute__((aligned(16))) float sD[2 * kKvWaves * BMQ];

  // Block order. Workgroup i runs on XCD i % 8. When the heads split evenly over the 8 XCDs,
  // each XCD takes heads / 8 heads of a sequence: first the key blocks that hold prefix keys
  // (their query loops are the long ones), one head after the other, so the blocks running
  // together on an XCD stream the same head's Q / dO tiles through its L2; then the window blocks.
  // Otherwise: key blocks outermost across heads, so the prefix blocks still start first.
  const int idx = blockIdx.x;
  int h, kblk, s;
  if (a.heads % 8 == 0) {
    const int per = a.heads * nkb;
    s = idx / per;
    const int i = idx - s * per, x = i % 8, j = i / 8, hg = a.heads / 8;
    const int P = min(nkb, max(0, (a.prefix_len[s] + BNK - 1) / BNK));
    if (j < hg * P) {
      h = x * hg + j / P;
      kblk = j % P;
    } else {
      const int w = nkb - P, jj = j - hg * P;
      h = x * hg + jj / w;
      kblk = P + jj % w;
    }
  } else {
    h = idx % a.heads;
    kblk = (idx / a.heads) % nkb;
    s = idx / (a.heads * nkb);
  }
  const int cu0 = a.cu_seqlens[s];
  const int S = a.cu_seqlens[s + 1] - cu0;
  // metadata check, as in the forward: the last key block of the grid covers the sequence end
  if (kblk == nkb - 1 && threadIdx.x == 0) {
    const int mm = a.prefix_len[s], nn = a.window[s];
    if (S < 0 || S > nkb * BNK || mm < 0 || mm > S || nn < 1) *a.err = 1;
  }
  const int k0 = kblk * BNK;
  if (k0 >= S) return;
  const int m = a.prefix_len[s];
  const int n = a.window[s];
  const bool pc = a.prefix_causal != 0;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int64_t rs = (int64_t)a.heads * kHeadDim;
  const int64_t hoff = ((int64_t)cu0 * a.heads + h) * kHeadDim;
  const uint16_t* qbase = a.q + hoff;
  const uint16_t* gbase = a.dout + hoff;
  const float* lse = a.work + h * (a.rows / a.heads) + cu0;  // lse * log2(e), head-major
  const float* dlt = lse + a.rows;                            // -delta

  const float c = a.scale_log2;
  const SwzLane sl_(lane);
  u32x4 kf[8], vf[8];
  // this lane's key as B operands (8 d-steps of 16 of its K and V rows)
  auto load_kv = [&](int key) {
    const int kc = min(key, S - 1);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      kf[st] = *reinterpret_cast<const u32x4*>(a.k + hoff + kc * rs + st * 16 + half * 8);
      vf[st] = *reinterpret_cast<const u32x4*>(a.v + hoff + kc * rs + st * 16 + half * 8);
    }
    // Materialise the operands here: the compiler then waits for these loads once, before the
    // loop, instead of inside it, where its wait would also cover the tile DMA in flight.
#pragma unroll
    for (int st = 0; st < 8; ++st) asm volatile("" : "+a"(kf[st]), "+a"(vf[st]));
  };
  // queries that see key kw: [lo, hi)
  auto key_range = [&](int key, int& lo, int& hi) {
    if (key >= S) {
      lo = hi = 0;
    } else if (key < m) {
      lo = pc ? key : 0;
      hi = S;
    } else {
      lo = key;
      hi = min(S, key + n);
    }
  };

  // The block that straddles the prefix end (m not a multiple of 128): its first hs key sets of
  // 32 hold the r = m mod 128 prefix keys, which every later query sees, while its other keys see
  // only their windows. Run as usual, one wave would stream all queries while three wait; instead
  // the four waves take one such key set at a time and a quarter of its query blocks each, from
  // private double-buffered 32-query tiles, and add their partial dK, dV through LDS. The main
  // loop below then handles the block's remaining (window-only) keys.
  const int r_pre = m % BNK;
  const bool boundary = r_pre > 0 && kblk == m / BNK;
  const int hs = boundary ? (r_pre + 31) / 32 : 0;
  for (int set = 0; set < hs; ++set) {
    const int ks0 = k0 + 32 * set;
    const int kws = ks0 + (lane & 31);
    load_kv(kws);
    int plo, phi;
    key_range(kws, plo, phi);
    const int slo = pc ? ks0 : 0;  // ks0 < m: a prefix key set
    const int nb = (S - slo + 31) / 32;
    const int per = (nb + kKvWaves - 1) / kKvWaves;
    const int b0 = min(nb, wave * per), b1 = min(nb, b0 + per);
    floatx16 dk[4], dv[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      zero16(dk[db]);
      zero16(dv[db]);
    }
    uint16_t* wq = sQ + wave * Q_TILE;  // this wave's two 32-row Q buffers
    uint16_t* wg = sG + wave * Q_TILE;
    float* wl = sL + wave * 2 * BMQ;    // and two 64-float lse / delta buffers
    float* wd = sD + wave * 2 * BMQ;
    auto issue_blk = [&](int b, int buf) {
      const int p0 = slo + 32 * b;
      dma4(lse + min(p0 + lane, S - 1), wl + buf * BMQ);
      dma4(dlt + min(p0 + lane, S - 1), wd + buf * BMQ);
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int row = 4 * g + (lane >> 4);
        const int64_t off = (int64_t)min(p0 + row, S - 1) * rs + 8 * ((lane & 15) ^ swz(row));
        dma16(qbase + off, wq + buf * 32 * kHeadDim + g * 4 * kHeadDim);
        dma16(gbase + off, wg + buf * 32 * kHeadDim + g * 4 * kHeadDim);
      }
    };
    constexpr int kBlkPieces = 18;
    if (b0 < b1) issue_blk(b0, 0);
    if (b0 + 1 < b1) issue_blk(b0 + 1, 1);
    for (int b = b0; b < b1; ++b) {
      const int buf = (b - b0) & 1;
      if (b + 1 < b1)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kBlkPieces) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      const uint16_t* q_t = wq + buf * 32 * kHeadDim;
      const uint16_t* g_t = wg + buf * 32 * kHeadDim;
      const float* l_t = wl + buf * BMQ;
      const float* d_t = wd + buf * BMQ;
      floatx16 sacc, dpacc;
      zero16(sacc);
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const float4 d4 = *reinterpret_cast<const float4*>(d_t + 8 * gg + 4 * half);
        dpacc[4 * gg + 0] = d4.x;  // -delta: the chain yields dP - delta
        dpacc[4 * gg + 1] = d4.y;
        dpacc[4 * gg + 2] = d4.z;
        dpacc[4 * gg + 3] = d4.w;
      }
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        sacc = mfma32(swz_ld_a(q_t, sl_, 0, st), kf[st], sacc);
        dpacc = mfma32(swz_ld_a(g_t, sl_, 0, st), vf[st], dpacc);
      }
      const int pb0 = slo + 32 * b;
      const uint32_t p_rel = (uint32_t)(pb0 + 4 * half - plo);
      const uint32_t p_width = (uint32_t)(phi - plo);
      float pr[16], ds[16];
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const float4 l4 = *reinterpret_cast<const float4*>(l_t + 8 * gg + 4 * half);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 4 * gg + i;
          const bool vis = p_rel + (uint32_t)(8 * gg + i) < p_width;
          pr[rr] = vis ? fast_exp2(fmaf(sacc[rr], c, -lv[i])) : 0.f;
          ds[rr] = pr[rr] * dpacc[rr];
        }
      }
      const u32x4 pb[2] = {pack_b(pr, 0), pack_b(pr, 1)};
      const u32x4 sb[2] = {pack_b(ds, 0), pack_b(ds, 1)};
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          dv[db] = mfma32(swz_ld_tr(g_t, sl_, 16 * st, db), pb[st], dv[db]);
          dk[db] = mfma32(swz_ld_tr(q_t, sl_, 16 * st, db), sb[st], dk[db]);
        }
      if (b + 2 < b1) {
        // every LDS read of this buffer has returned before the copy overwrites it
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue_blk(b + 2, buf);
      }
    }
    // add the four partial dK^T, dV^T (this wave's registers; same lane layout in every wave)
    __syncthreads();
    float* pk = reinterpret_cast<float*>(wq);  // 16 KB: 64 registers x 64 lanes
    float* pv = reinterpret_cast<float*>(wg);
    if (wave > 0) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          pk[(db * 16 + i) * 64 + lane] = dk[db][i];
          pv[(db * 16 + i) * 64 + lane] = dv[db][i];
        }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 1; w < kKvWaves; ++w) {
        const float* ok = reinterpret_cast<const float*>(sQ + w * Q_TILE);
        const float* ov = reinterpret_cast<const float*>(sG + w * Q_TILE);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            dk[db][i] += ok[(db * 16 + i) * 64 + lane];
            dv[db][i] += ov[(db * 16 + i) * 64 + lane];
          }
      }
      if (kws < S) {
        const int64_t row = ((int64_t)(cu0 + kws) * a.heads + h) * kHeadDim;
        store_row128<OUT>(reinterpret_cast<OUT*>(a.dk) + row, dk, a.scale, half);
        store_row128<OUT>(reinterpret_cast<OUT*>(a.dv) + row, dv, 1.f, half);
      }
    }
    __syncthreads();
  }
  if (hs == kKvWaves) return;  // the whole block held prefix keys (uniform)

  // this lane's key (none for the waves whose key sets the split above covered)
  const int wk0 = k0 + wave * 32;
  const int kw = wave < hs ? S : wk0 + (lane & 31);
  load_kv(kw);
  int plo, phi;
  key_range(kw, plo, phi);
  const int kfirst = k0 + 32 * hs;  // first key the loop below owns
  const int klast = min(k0 + BNK, S) - 1;
  const int qlo = kfirst < m ? (pc ? kfirst : 0) : kfirst;
  const int qhi = kfirst < m ? S : min(S, klast + n);
  const int ntiles = (qhi - qlo + BMQ - 1) / BMQ;
  const bool wave_pre = wave >= hs && wk0 + 32 <= min(m, S);  // all the wave's keys are prefix keys

  floatx16 dk[4], dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    zero16(dk[db]);
    zero16(dv[db]);
  }

  // copy tile j into buffer set b (= j % 4)
  auto issue_to = [&](int j, int b) {
    dma_qtile(sQ + b * Q_TILE, sG + b * Q_TILE, sL + b * BMQ, sD + b * BMQ, qbase, gbase, lse,
              dlt, rs, qlo + j * BMQ, S - 1, wave, lane);
  };
  auto issue = [&](int j) { issue_to(j, j & 3); };

  // Scores of block b (queries qlo + 32 b + ...) that this lane's key cannot see set to -inf,
  // where the block is not fully visible (uniform per wave); P and dS are then exactly zero.
  // Accumulator register r holds query pb0 + 8 (r / 4) + 4 half + r % 4.
  auto mask_block = [&](floatx16& sc, int b) {
    const int pb0 = qlo + 32 * b;
    const bool masked = !(wave_pre && pb0 + 32 <= S && (!pc || pb0 >= wk0 + 31));
    if (masked) {
      const uint32_t p_rel = (uint32_t)(pb0 + 4 * half - plo);
      const uint32_t p_width = (uint32_t)(phi - plo);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sc[r] = p_rel + (uint32_t)(8 * (r >> 2) + (r & 3)) < p_width ? sc[r] : -INFINITY;
    }
  };

  // One step: S and dP - delta of the next block (rows rn of tile buffers qn / gn / dn_) into
  // sn / dn under P, dS of the current block (scores sc, dc; rows rc of qc / gc / lc), then
  // dV^T += dO^T P and dK^T += Q^T dS for the current block. With the Guarded tag, the last S and
  // dP MFMAs are followed by the wait states their results need: the compiler moves sn / dn to
  // other registers right after them in the single-tile loop and at the unrolled loop's back
  // edge. Elsewhere they stay in place until the next step reads them, 16 MFMAs later.
  auto step = [&](auto guard, floatx16& sc, floatx16& dc, floatx16& sn, floatx16& dn,
                  const uint16_t* qn,
                  const uint16_t* gn, const float* dn_, int rn, const uint16_t* qc,
                  const uint16_t* gc, const float* lc, int rc) {
    float4 l4[4], d4[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      l4[g] = *reinterpret_cast<const float4*>(lc + rc + 8 * g + 4 * half);
      d4[g] = *reinterpret_cast<const float4*>(dn_ + rn + 8 * g + 4 * half);
    }
    u32x4 fq[3], fg[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      fq[i] = swz_ld_a(qn, sl_, rn, i);
      fg[i] = swz_ld_a(gn, sl_, rn, i);
    }
    FENCE();
#pragma unroll
    for (int g = 0; g < 4; ++g) {  // dP accumulates on top of -delta: the chain yields dP - delta
      dn[4 * g + 0] = d4[g].x;
      dn[4 * g + 1] = d4[g].y;
      dn[4 * g + 2] = d4[g].z;
      dn[4 * g + 3] = d4[g].w;
    }
    float pr[16], ds[16];
    u32x4 pb[2], sb[2], tg[2], tq[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i == 0) {
        mfma_vacc_zero(sn, fq[0], kf[0]);
        mfma_vacc_first(dn, fg[0], vf[0]);
      } else if (i < 7 || !decltype(guard)::value) {
        mfma_vacc(sn, fq[i % 3], kf[i]);
        mfma_vacc(dn, fg[i % 3], vf[i]);
      } else {
        mfma_vacc_last2(sn, fq[i % 3], kf[i], dn, fg[i % 3], vf[i]);
      }
      if (i + 3 < 8) {
        fq[i % 3] = swz_ld_a(qn, sl_, rn, i + 3);
        fg[i % 3] = swz_ld_a(gn, sl_, rn, i + 3);
      }
#pragma unroll
      for (int e = 2 * i; e < 2 * i + 2; ++e) {
        const float lv = (e & 3) == 0 ? l4[e >> 2].x : (e & 3) == 1 ? l4[e >> 2].y
                                                      : (e & 3) == 2 ? l4[e >> 2].z : l4[e >> 2].w;
        pr[e] = fast_exp2(fmaf(sc[e], c, -lv));
        ds[e] = pr[e] * dc[e];
      }
      if (i == 4) {
        pb[0] = pack_b(pr, 0);
        sb[0] = pack_b(ds, 0);
      }
      if (i >= 8 - 2) {  // transposed operands of the first products of the second half
        const int k = i - (8 - 2);  // pair k: d block k / 2, key step k % 2
        tg[k] = swz_ld_tr(gc, sl_, rc + 16 * (k & 1), k >> 1);
        tq[k] = swz_ld_tr(qc, sl_, rc + 16 * (k & 1), k >> 1);
      }
      FENCE();
    }
    pb[1] = pack_b(pr, 1);
    sb[1] = pack_b(ds, 1);
    FENCE();
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int db = k >> 1, st = k & 1;
      dv[db] = mfma32(tg[k % 2], pb[st], dv[db]);
      dk[db] = mfma32(tq[k % 2], sb[st], dk[db]);
      if (k + 2 < 8) {
        const int kk = k + 2;
        tg[k % 2] = swz_ld_tr(gc, sl_, rc + 16 * (kk & 1), kk >> 1);
        tq[k % 2] = swz_ld_tr(qc, sl_, rc + 16 * (kk & 1), kk >> 1);
      }
      FENCE();
    }
  };

  issue(0);
  if (ntiles > 1) issue(1);
  if (ntiles > 2) issue(2);
  if (ntiles > 2)
    dma_wait_barrier<2 * kKvPieces>();
  else if (ntiles > 1)
    dma_wait_barrier<kKvPieces>();
  else
    dma_wait_barrier<0>();

  // block 0's S and dP - delta
  floatx16 s0, d0, s1, d1;
  {
    zero16(s0);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 d = *reinterpret_cast<const float4*>(sD + 8 * g + 4 * half);
      d0[4 * g + 0] = d.x;  // -delta
      d0[4 * g + 1] = d.y;
      d0[4 * g + 2] = d.z;
      d0[4 * g + 3] = d.w;
    }
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      s0 = mfma32(swz_ld_a(sQ, sl_, 0, st), kf[st], s0);
      d0 = mfma32(swz_ld_a(sG, sl_, 0, st), vf[st], d0);
    }
    mask_block(s0, 0);
  }

  int j = 0;
  // four tiles per iteration while every wait and copy of them is the steady-state one, so that
  // every LDS buffer offset is a constant
  for (; j + 7 <= ntiles; j += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int b = u, bn = (u + 1) & 3;
      const uint16_t* q_j = sQ + b * Q_TILE;
      const uint16_t* g_j = sG + b * Q_TILE;
      step(Unguarded{}, s0, d0, s1, d1, q_j, g_j, sD + b * BMQ, 32, q_j, g_j, sL + b * BMQ, 0);
      mask_block(s1, 2 * (j + u) + 1);
      dma_wait_barrier<kKvPieces>();
      issue_to(j + u + 3, (u + 3) & 3);
      if (u < 3)
        step(Unguarded{}, s1, d1, s0, d0, sQ + bn * Q_TILE, sG + bn * Q_TILE, sD + bn * BMQ, 0,
             q_j, g_j, sL + b * BMQ, 32);
      else  // the loop's last step: its results cross the loop's back edge
        step(Guarded{}, s1, d1, s0, d0, sQ + bn * Q_TILE, sG + bn * Q_TILE, sD + bn * BMQ, 0, q_j,
             g_j, sL + b * BMQ, 32);
      mask_block(s0, 2 * (j + u) + 2);
    }
  }
  for (; j < ntiles; ++j) {
    const int b = j & 3, bn = (j + 1) & 3;
    const uint16_t* q_j = sQ + b * Q_TILE;
    const uint16_t* g_j = sG + b * Q_TILE;
    step(Guarded{}, s0, d0, s1, d1, q_j, g_j, sD + b * BMQ, 32, q_j, g_j, sL + b * BMQ, 0);
    mask_block(s1, 2 * j + 1);
    // tile j + 1 must have landed (tile j + 2's copy may still be in flight); past this barrier
    // every wave is done with tile j - 1, whose buffers take tile j + 3
    if (j + 2 < ntiles)
      dma_wait_barrier<kKvPieces>();
    else
      dma_wait_barrier<0>();
    if (j + 3 < ntiles) issue(j + 3);
    step(Guarded{}, s1, d1, s0, d0, sQ + bn * Q_TILE, sG + bn * Q_TILE, sD + bn * BMQ, 0, q_j,
         g_j, sL + b * BMQ, 32);
    if (j + 1 < ntiles) mask_block(s0, 2 * j + 2);
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
#ifndef RSWA_DQ_SCHED
#define RSWA_DQ_SCHED 0  // > 0: fragment reads kept this far ahead of the score MFMAs
#endif
#ifndef RSWA_DQ_WAVES
#define RSWA_DQ_WAVES 8  // waves per workgroup, 32 queries each
#endif
constexpr int kDqWaves = RSWA_DQ_WAVES;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int BNQ = 32 * kDqWaves;                  // queries per workgroup
constexpr int BN = 64;                              // keys per tile
constexpr int K_TILE = BN * kHeadDim;               // swizzled K / V tile (bf16 elements)

constexpr int kKeyGroupsPerWave = BN / 4 / kDqWaves;  // 4-row (1 KB) groups per wave
constexpr int kDqPieces = 2 * kKeyGroupsPerWave;       // 16-byte DMA loads per wave per tile

// Keys k0 .. k0 + 63 of K and V (rows clamped to kmax) copied by LDS DMA into one buffer pair.
__device__ __forceinline__ void dma_ktile(uint16_t* sk, uint16_t* sv, const uint16_t* kbase,
                                          const uint16_t* vbase, int64_t rs, int k0, int kmax,
                                          int wave, int lane) {
#pragma unroll
  for (int u = 0; u < kKeyGroupsPerWave; ++u) {
    const int grp = wave * kKeyGroupsPerWave + u;
    const int row = 4 * grp + (lane >> 4);
    const int c = (lane & 15) ^ swz(row);
    const int64_t off = (int64_t)min(k0 + row, kmax) * rs + c * 8;
    dma16(kbase + off, sk + grp * 4 * kHeadDim);
    dma16(vbase + off, sv + grp * 4 * kHeadDim);
  }
}

template <typename OUT>
__global__ __launch_bounds__(kDqThreads) void dq_kernel(BwdArgs a) {
  // four buffer pairs: the DMA for tile j + 3 runs while tile j is computed
  __shared__ __attribute__((aligned(16))) uint16_t sK[4 * K_TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[4 * K_TILE];

  // XCD-aware tile order (as in the forward): workgroup i runs on XCD i % 8, so each XCD takes a
  // contiguous run of (query tile, head) pairs and one head's K / V tiles stay in its L2.
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
    if (S < 0 || S > (int)gridDim.x * BNQ || mm < 0 || mm > S || nn < 1) *a.err = 1;
  }
  const int q0 = bx * BNQ;
  if (q0 >= S) return;
  const int q1 = min(q0 + BNQ, S);
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

  // this lane's query, its Q and dO rows as B operands, its lse (log2 domain) and delta
  const int p = q0 + wave * 32 + lq;
  const int pq = min(p, S - 1);
  u32x4 qf[8], gf[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    qf[st] = *reinterpret_cast<const u32x4*>(a.q + hoff + pq * rs + st * 16 + half * 8);
    gf[st] = *reinterpret_cast<const u32x4*>(a.dout + hoff + pq * rs + st * 16 + half * 8);
  }
  const int64_t prow = h * (a.rows / a.heads) + cu0 + pq;  // head-major work rows
  float lse2 = a.work[prow];
  float dlt = a.work[a.rows + prow];  // -delta
  // Materialise the operands here: the compiler then waits for these loads once, before the
  // loop, instead of inside it, where its wait would also cover the tile DMA in flight.
#pragma unroll
  for (int st = 0; st < 8; ++st) asm volatile("" : "+v"(qf[st]), "+v"(gf[st]));
  asm volatile("" : "+v"(lse2), "+v"(dlt));

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
  const SwzLane sl_(lane);

  // copy tile j into buffer pair b (= j % 4)
  auto issue_to = [&](int j, int b) {
    dma_ktile(sK + b * K_TILE, sV + b * K_TILE, kbase, vbase, rs, tstart(j), S - 1, wave, lane);
  };
  auto issue = [&](int j) { issue_to(j, j % 4); };
  issue(0);
  if (ntiles > 1) issue(1);
  if (ntiles > 2) issue(2);
  if (ntiles > 2)
    dma_wait_barrier<2 * kDqPieces>();
  else if (ntiles > 1)
    dma_wait_barrier<kDqPieces>();
  else
    dma_wait_barrier<0>();

  // One 32-key block of the tile in LDS buffers (sk, sv): S^T = K Q^T and dP^T = V dO^T (keys in
  // accumulator rows, this lane's query in the column), dS^T in registers, dQ^T += K^T dS^T.
  // A key is visible iff it lies in [lo, hi], tested as one unsigned range check.
  auto kblock = [&](const uint16_t* sk, const uint16_t* sv, int kb, int k0, int lo,
                    int hi, bool masked) {
    __builtin_amdgcn_sched_barrier(0);  // blocks do not interleave: registers stay bounded
    floatx16 sacc, dpacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) dpacc[r] = dlt;  // -delta: the chain yields dP - delta
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const u32x4 ka = swz_ld_a(sk, sl_, kb * 32, st);
      sacc = mfma32(ka, qf[st], st == 0 ? floatx16{} : sacc);  // the first starts from 0
    }
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const u32x4 va = swz_ld_a(sv, sl_, kb * 32, st);
      dpacc = mfma32(va, gf[st], dpacc);
    }
#if RSWA_DQ_SCHED
    // keep RSWA_DQ_SCHED fragment reads in flight ahead of the score chains
    __builtin_amdgcn_sched_group_barrier(0x100, RSWA_DQ_SCHED, 0);
#pragma unroll
    for (int i = 0; i < 16 - RSWA_DQ_SCHED; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, RSWA_DQ_SCHED, 0);
#endif
    // accumulator register r: key k0 + kb*32 + 8 (r / 4) + 4 half + r % 4, query p
    const uint32_t k_rel = (uint32_t)(k0 + kb * 32 + 4 * half - lo);
    const uint32_t k_width = (uint32_t)max(hi - lo + 1, 0);
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] = fast_exp2(fmaf(sacc[r], c, -lse2)) * dpacc[r];
    if (masked) {  // uniform: only tiles that are not wholly visible
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ds[r] = (k_rel + (uint32_t)(8 * (r >> 2) + (r & 3)) < k_width) ? ds[r] : 0.f;
    }
    const u32x4 sb[2] = {pack_b(ds, 0), pack_b(ds, 1)};
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4 ka = swz_ld_tr(sk, sl_, kb * 32 + 16 * st, db);
        dq[db] = mfma32(ka, sb[st], dq[db]);
      }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Leading tiles that need no element mask (inside the prefix, and below the diagonal of a
  // causal prefix) run a loop without mask tests or end-of-loop cases.
  int n_plain = min(m / BN, n_pre);
  if (pc && q0 < m) n_plain = min(n_plain, (q0 + 1) / BN);
  const int j_plain = min(n_plain, ntiles - 3);
  int j = 0;
  // four tiles per iteration, so that every LDS buffer offset is a constant
  for (; j + 4 <= j_plain; j += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      issue_to(j + u + 3, (u + 3) % 4);
      const uint16_t* sk = sK + u * K_TILE;
      const uint16_t* sv = sV + u * K_TILE;
      kblock(sk, sv, 0, 0, 0, 0, false);
      kblock(sk, sv, 1, 0, 0, 0, false);
      dma_wait_barrier<2 * kDqPieces>();
    }
  }
  for (; j < j_plain; ++j) {
    const int buf = j % 4;
    issue(j + 3);
    const uint16_t* sk = sK + buf * K_TILE;
    const uint16_t* sv = sV + buf * K_TILE;
    kblock(sk, sv, 0, 0, 0, 0, false);
    kblock(sk, sv, 1, 0, 0, 0, false);
    dma_wait_barrier<2 * kDqPieces>();
  }
  for (; j < ntiles; ++j) {
    const int buf = j % 4;
    if (j + 3 < ntiles) issue(j + 3);
    const uint16_t* sk = sK + buf * K_TILE;
    const uint16_t* sv = sV + buf * K_TILE;
    const int k0 = tstart(j);
    const bool is_pre = j < n_pre;
    const int lo = is_pre ? 0 : win_lo;
    const int hi = is_pre ? pre_hi : p;
    // uniform per tile: prefix tiles that every query of the workgroup sees whole need no mask
    const bool masked = is_pre ? (k0 + BN > m || (pc && q0 < m && k0 + BN - 1 > q0)) : true;
    kblock(sk, sv, 0, k0, lo, hi, masked);
    kblock(sk, sv, 1, k0, lo, hi, masked);
    if (j + 3 < ntiles)
      dma_wait_barrier<2 * kDqPieces>();
    else if (j + 2 < ntiles)
      dma_wait_barrier<kDqPieces>();
    else
      dma_wait_barrier<0>();
  }

  if (p < q1)
    store_row128<OUT>(reinterpret_cast<OUT*>(a.dq) + ((int64_t)(cu0 + p) * a.heads + h) * kHeadDim,
                      dq, a.scale, half);
}

}  // namespace

hipError_t launch_prefill_bwd(const BwdArgs& a, int out_f32, int grad_f32, hipStream_t s) {
  const int64_t rows = a.rows, total = a.rows / a.heads;
  if (rows > 0) {
    const dim3 g((unsigned)((total + 31) / 32 * a.heads));
    if (out_f32)
      hipLaunchKernelGGL(delta_kernel<float>, g, dim3(256), 0, s,
                         reinterpret_cast<const float*>(a.out), a.dout, a.lse, a.work, total,
                         a.heads);
    else
      hipLaunchKernelGGL(delta_kernel<uint16_t>, g, dim3(256), 0, s,
                         reinterpret_cast<const uint16_t*>(a.out), a.dout, a.lse, a.work, total,
                         a.heads);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 gq((a.max_seqlen + BNQ - 1) / BNQ, a.heads, a.nseq);
  const int nkb = (a.max_seqlen + BNK - 1) / BNK;
  const dim3 gkv((unsigned)nkb * a.heads * a.nseq);
  if (grad_f32)
    hipLaunchKernelGGL(dkdv_kernel<float>, gkv, dim3(kKvThreads), 0, s, a, nkb);
  else
    hipLaunchKernelGGL(dkdv_kernel<uint16_t>, gkv, dim3(kKvThreads), 0, s, a, nkb);
  if (grad_f32)
    hipLaunchKernelGGL(dq_kernel<float>, gq, dim3(kDqThreads), 0, s, a);
  else
    hipLaunchKernelGGL(dq_kernel<uint16_t>, gq, dim3(kDqThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace rswa
