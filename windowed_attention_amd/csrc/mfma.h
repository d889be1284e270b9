// gfx950 matrix-core and LDS helpers shared by the attention kernels of the teacher-forced pass.
//
// v_mfma_f32_32x32x16_bf16 operand layouts (lane l, l32 = l % 32, half = l / 32):
//   A (32 x 16): lane l holds row l32, columns 8 half .. 8 half + 7;
//   B (16 x 32): lane l holds column l32, rows 8 half .. 8 half + 7;
//   C (32 x 32): accumulator register r of lane l holds column l32, row 8 (r / 4) + 4 half + r % 4.
#pragma once

#include "device.h"

namespace rswa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native vector: stays in VGPRs
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx16 mfma32(const u32x4& a, const u32x4& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ void zero16(floatx16& x) {
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = 0.f;
}

// two floats -> packed bf16 pair (round to nearest even), low half first
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2v_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Accumulator registers 8 st .. 8 st + 7 rounded to bf16: the B operand of a product whose
// contraction runs over the accumulator's rows (step st of two 16-row steps).
__device__ __forceinline__ u32x4 pack_b(const float (&x)[16], int st) {
  return u32x4{pack_bf16(x[8 * st + 0], x[8 * st + 1]), pack_bf16(x[8 * st + 2], x[8 * st + 3]),
               pack_bf16(x[8 * st + 4], x[8 * st + 5]), pack_bf16(x[8 * st + 6], x[8 * st + 7])};
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): within each group of 16 lanes, output lane i
// gets element i % 4 of the 8-byte chunks that lanes 4j + i / 4 (j = 0..3) point at. With lane
// 4j + q pointing at X[r0 + j][c0 + 4q .. +3], lane i receives X[r0 .. r0 + 3][c0 + i]: four
// consecutive rows of its own column, i.e. half of a transposed MFMA operand.
__device__ __forceinline__ u32x2 ld_tr(const uint16_t* p) {
  const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (v4i16_t __attribute__((address_space(3)))*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// A operand X^T (32 columns c0 .. c0 + 31 of a row-major LDS tile, 16 rows) for a product whose
// B operand comes from accumulator registers 8 st .. 8 st + 7 (see pack_b): lane l gets column
// c0 + l % 32 at rows r0 + 16 st + 8 (e / 4) + 4 half + e % 4, e = 0..7, which is the row order
// of those accumulator registers. `base` = tile + (((l % 16) / 4) + 4 half) * stride
// + 16 ((l / 16) % 2) + 4 (l % 4), computed once per kernel.
__device__ __forceinline__ u32x4 ld_tr_op(const uint16_t* base, int stride, int r0, int c0) {
  const uint16_t* p = base + r0 * stride + c0;
  const u32x2 lo = ld_tr(p);
  const u32x2 hi = ld_tr(p + 8 * stride);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}
__device__ __forceinline__ const uint16_t* tr_base(const uint16_t* tile, int stride, int lane) {
  return tile + (((lane & 15) >> 2) + 4 * (lane >> 5)) * stride + 16 * ((lane >> 4) & 1) +
         4 * (lane & 3);
}

// 128-wide bf16 tile (rows of 256 bytes, no padding) whose 16-byte chunks are XOR-swizzled per row:
// chunk c of row r is stored at chunk c ^ swz(r), swz(r) = 4 (r % 4) + (r / 4) % 4. The straight
// 16-byte operand read (16 consecutive rows, one chunk) and the transposing read (4 consecutive rows
// x 4 chunks) then both cover 16 distinct 16-byte bank groups of LDS's 256-byte bank row, so a
// tile that is read both ways has no bank conflicts (a padded row stride serves only one of them).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// element offset of chunk c (8 bf16) of row r
__device__ __forceinline__ int swz_chunk(int r, int c) { return r * kHeadDim + 8 * (c ^ swz(r)); }

// Per-lane constants of the operand reads from a swizzled tile.
struct SwzLane {
  int a_off;  // straight read: row lq
  int a_f;    // swz(lq % 16)
  int a_half;
  int t_off;  // transposing read: row j = (lane % 16) / 4 + 4 half, element 4 (lane % 2)
  int t_f;    // swz(j)
  int t_x;    // chunk within a 4-chunk column block: 2 ((lane / 16) % 2) + (lane % 4) / 2
  __device__ __forceinline__ explicit SwzLane(int lane) {
    const int lq = lane & 31, half = lane >> 5;
    const int j = ((lane & 15) >> 2) + 4 * half;
    a_off = lq * kHeadDim;
    a_f = swz(lq & 15);
    a_half = half;
    t_off = j * kHeadDim + 4 * (lane & 1);
    t_f = swz(j);
    t_x = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  }
};

// Straight A operand (32 rows r0 .. r0 + 31, r0 a multiple of 16; columns 16 st .. 16 st + 15).
__device__ __forceinline__ u32x4 swz_ld_a(const uint16_t* tile, const SwzLane& L, int r0, int st) {
  return *reinterpret_cast<const u32x4*>(tile + r0 * kHeadDim + L.a_off +
                                         8 * ((2 * st + L.a_half) ^ L.a_f));
}

// Transposed operand of ld_tr_op from a swizzled tile: columns 32 db + lane % 32, rows
// r0 + 8 (e / 4) + 4 half + e % 4 (r0 a multiple of 16). Rows j + 8 have swz(j + 8) = swz(j) ^ 2.
__device__ __forceinline__ u32x4 swz_ld_tr(const uint16_t* tile, const SwzLane& L, int r0, int db) {
  const uint16_t* p = tile + r0 * kHeadDim + L.t_off;
  const u32x2 lo = ld_tr(p + 8 * ((4 * db + L.t_x) ^ L.t_f));
  const u32x2 hi = ld_tr(p + 8 * kHeadDim + 8 * ((4 * db + L.t_x) ^ L.t_f ^ 2));
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// gfx950 LDS DMA (global_load_lds_dwordx4 / _dword): each lane copies 16 (4) bytes from its
// global address straight into LDS, without passing through registers; the wave's pieces land
// contiguously at `lds` (wave-uniform, placed in M0), lane L at byte 16 L (4 L). Completion is
// counted by the wave's vector-memory counter and waited for with dma_wait_barrier. The loads are
// issued from inline assembly so that the compiler, which cannot tell the DMA's LDS target from
// the buffers being read, does not wait for every DMA in flight before each LDS read.
__device__ __forceinline__ uint32_t lds_addr(const void* lds) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds);
}
// The DMA takes its LDS address from M0; a scalar write of M0 needs one wait state before an LDS
// DMA reads it (the `s_nop 0`, which the compiler would insert between instructions it knows).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is reserved; it is set right here
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
               "s"(lds_addr(lds))
               : "memory", "m0");
}
// The same copy from a wave-uniform base address (SGPR pair) plus a per-lane 32-bit byte offset:
// the address arithmetic of a tile then runs on the scalar unit.
// `lds` is an LDS byte address (lds_addr of the destination), wave-uniform.
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off),
               "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g),
               "s"(lds_addr(lds))
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N of this wave's vector-memory loads are outstanding (loads complete in
// issue order), then join the workgroup barrier. Written out because __syncthreads' fence would
// also wait for the DMA loads issued for later tiles.
template <int N>
__device__ __forceinline__ void dma_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <typename OUT>
__device__ __forceinline__ void store_out4(OUT* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store_out4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store_out4<uint16_t>(uint16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2*>(p) = u32x2{f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16),
                                       f32_to_bf16_bits(c) | (f32_to_bf16_bits(d) << 16)};
}

// Store a transposed 128-wide accumulator row (four 32-row blocks of C^T, this lane's column)
// times `mul`: dims db * 32 + 8 g + 4 half + (0..3).
template <typename OUT>
__device__ __forceinline__ void store_row128(OUT* row, const floatx16 (&acc)[4], float mul, int half) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      store_out4<OUT>(row + db * 32 + 8 * g + 4 * half, acc[db][4 * g] * mul,
                      acc[db][4 * g + 1] * mul, acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul);
}

// max / sum over the two lane halves holding the same C column (lanes l and l ^ 32)
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace rswa
