// Device helpers shared by the gfx950 kernels: bf16 packing, DPP row reductions, exp2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rswa {

constexpr int kHeadDim = 128;     // D: the only head size the kernels are built for
constexpr int kWave = 64;         // CDNA wavefront width
constexpr float kNegBig = -1e30f; // finite "minus infinity" for running maxima (keeps
                                  // exp2(m_old - m_new) = 1 while a row has seen nothing)

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Raw v_exp_f32 (2^x); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of a DPP row; every lane of the row receives the total.
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  x += dpp_mov<0x140>(x);
  return x;
}

// Sum over 32 consecutive lanes (two DPP rows joined with a ds_swizzle xor-16 exchange).
__device__ __forceinline__ float lane32_sum(float x) {
  x = row16_sum(x);
  x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
  return x;
}

// Store one float to an output element of type OUT (uint16_t = bf16 bits, or float).
__device__ __forceinline__ void store_out(uint16_t* p, float x) { *p = (uint16_t)f32_to_bf16_bits(x); }
__device__ __forceinline__ void store_out(float* p, float x) { *p = x; }

}  // namespace rswa
