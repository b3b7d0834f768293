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
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw (stride 0) buffer resource over `bytes` bytes at p: loads at an offset past the end
// return zeros.  Word 3 is the gfx9 default (32-bit data format, no swizzle).
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

#define FLEXQ_WAVE 64

namespace flexq {

// 4-bit weight layout (flexq_w4): rows in blocks of 128; within a block, k-tile kt (64
// columns = one quantization group per row) holds the block's 128 x 32 bytes of codes
// contiguously (4 KiB), and its 128 (offset, scale) words contiguously, so a k-tile of
// any run of rows is read in whole cache lines.
constexpr int kW4BlockRows = 128;
constexpr int kW4TileBytes = kW4BlockRows * 32;
__host__ __device__ __forceinline__ int64_t w4_code_off(int64_t row, int64_t kt, int64_t KT) {
  return ((row >> 7) * KT + kt) * kW4TileBytes + (row & 127) * 32;   // bytes
}
__host__ __device__ __forceinline__ int64_t w4_param_idx(int64_t row, int64_t kt, int64_t KT) {
  return ((row >> 7) * KT + kt) * kW4BlockRows + (row & 127);       // 32-bit words
}

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

// Exact fp16 values of the codes in two bytes of `t` (bytes 0-1, or 2-3 when HI): a
// code zero-extended to a byte is the OCP FP8 E4M3 encoding of c * 2^-9 (subnormal
// for c < 8, exponent field 1 for c >= 8), so the scaled FP8 -> F16 convert with
// scale 2^9 returns c itself, with no rounding.
template <bool HI>
__device__ __forceinline__ f16x2 code_pair_f16(uint32_t t) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(t, 512.0f, HI);
}

// Spread 8 packed 4-bit codes (one 32-bit word, element 2j in the low nibble of byte
// j) to one code per byte: t0 = (c0, c1, c2, c3), t1 = (c4, c5, c6, c7).
__device__ __forceinline__ void codes_to_bytes(uint32_t w, uint32_t& t0, uint32_t& t1) {
  const uint32_t lo = w & 0x0F0F0F0Fu;          // c0 c2 c4 c6 in bytes 0..3
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // c1 c3 c5 c7
  // perm(S0 = hi, S1 = lo): selector bytes 0-3 pick lo bytes, 4-7 pick hi bytes
  t0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  t1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// The 4-bit weight layout keeps the eight codes of each 32-bit word in the order a
// spread to bytes needs no permute: byte j holds code j (low nibble) and code j + 4
// (high nibble).  w4_word_from_codes converts a word from the packed order above.
__device__ __forceinline__ uint32_t w4_word_from_codes(uint32_t w) {
  uint32_t t0, t1;
  codes_to_bytes(w, t0, t1);
  return t0 | (t1 << 4);
}
__device__ __forceinline__ void w4_word_to_bytes(uint32_t w, uint32_t& t0, uint32_t& t1) {
  t0 = w & 0x0F0F0F0Fu;
  t1 = (w >> 4) & 0x0F0F0F0Fu;
}

// The four exact code pairs (c_2j, c_2j+1), j = 0..3, of one packed word.
__device__ __forceinline__ void codes_to_pairs(uint32_t w, f16x2 out[4]) {
  uint32_t t0, t1;
  codes_to_bytes(w, t0, t1);
  out[0] = code_pair_f16<false>(t0);
  out[1] = code_pair_f16<true>(t0);
  out[2] = code_pair_f16<false>(t1);
  out[3] = code_pair_f16<true>(t1);
}

// The same for a word of the weight layout.
__device__ __forceinline__ void w4_word_to_pairs(uint32_t w, f16x2 out[4]) {
  uint32_t t0, t1;
  w4_word_to_bytes(w, t0, t1);
  out[0] = code_pair_f16<false>(t0);
  out[1] = code_pair_f16<true>(t0);
  out[2] = code_pair_f16<false>(t1);
  out[3] = code_pair_f16<true>(t1);
}

// Weight dequantization of one code pair: fp16(c * s + m) with a single rounding
// (fused multiply-add in fp16 of exact operands).
__device__ __forceinline__ f16x2 dequant_pair(f16x2 c, f16x2 s2, f16x2 m2) {
  return __builtin_elementwise_fma(c, s2, m2);
}

}  // namespace flexq

#define FLEXQ_LAUNCH_CHECK()                               \
  do {                                                     \
    if (hipGetLastError() != hipSuccess) return FLEXQ_ERR_DEVICE; \
  } while (0)
