// Shared device helpers for the flexq HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "flexq.h"

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define FLEXQ_WAVE 64

namespace flexq {

__device__ __forceinline__ f16 h_from_bits(uint16_t b) { return __builtin_bit_cast(f16, b); }
__device__ __forceinline__ uint16_t bits_from_h(f16 h) { return __builtin_bit_cast(uint16_t, h); }
__device__ __forceinline__ f16x2 h2_from_u32(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t u32_from_h2(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }

// DPP lane moves (row = 16 lanes).  quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_half_mirror (lane i <-> 7-i inside each 8-lane half row) = 0x141.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

// Reductions over aligned groups of 8 lanes (every lane gets the result).
__device__ __forceinline__ float oct_min(float v) {
  v = fminf(v, dpp_f32<0xB1>(v));
  v = fminf(v, dpp_f32<0x4E>(v));
  v = fminf(v, dpp_f32<0x141>(v));
  return v;
}
__device__ __forceinline__ float oct_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Expand 8 packed 4-bit codes (one 32-bit word, element 2j in the low nibble of
// byte j) to four fp16 pairs holding (1024 + c): the code sits in the low mantissa
// bits of 0x6400 = 1024.0.  Pair j holds elements (2j, 2j+1).
__device__ __forceinline__ void codes_to_magic_pairs(uint32_t w, uint32_t out[4]) {
  const uint32_t lo = w & 0x0F0F0F0Fu;          // c0 c2 c4 c6 in bytes 0..3
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // c1 c3 c5 c7
  // perm(S0=hi, S1=lo): selector bytes 0-3 pick lo bytes, 4-7 pick hi bytes, 0x0c -> 0
  out[0] = __builtin_amdgcn_perm(hi, lo, 0x0c040c00u) | 0x64006400u;
  out[1] = __builtin_amdgcn_perm(hi, lo, 0x0c050c01u) | 0x64006400u;
  out[2] = __builtin_amdgcn_perm(hi, lo, 0x0c060c02u) | 0x64006400u;
  out[3] = __builtin_amdgcn_perm(hi, lo, 0x0c070c03u) | 0x64006400u;
}

// Weight dequantization of one code pair: fp16(c * s + m) with a single rounding
// (fused multiply-add in fp16; c is exact after removing the 1024 bias).
__device__ __forceinline__ f16x2 dequant_pair(uint32_t magic_pair, f16x2 s2, f16x2 m2) {
  f16x2 c = h2_from_u32(magic_pair) - (f16x2){(f16)1024.0f, (f16)1024.0f};
  return __builtin_elementwise_fma(c, s2, m2);
}

}  // namespace flexq

#define FLEXQ_LAUNCH_CHECK()                               \
  do {                                                     \
    if (hipGetLastError() != hipSuccess) return FLEXQ_ERR_DEVICE; \
  } while (0)
