// Device-side group quantizer shared by the standalone quantize kernel, the prefill
// attention's KV store and the decode attention's append.
//
// A 64-element group is held by LPG consecutive lanes (LPG = 1, 4 or 8), each lane
// holding E = 64 / LPG consecutive elements.  Arithmetic follows the compression
// step of the FlexGen walkthrough, section 6.3 (4 bits, group 64, asymmetric
// min/max), in fp32 with a fixed sequence so that codes are reproducible:
//   step   = fp16(fl32(max - min) / 15)   (0 if max == min; 2^-24 if it underflows)
//   code   = clamp(rne(fl32(x - min) * fl32(1 / step)), 0, 15)
//   offset = min (a zero minimum stored as +0)
// Inputs are finite (the entry points require it).
#pragma once

#include "common.h"

namespace flexq {

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// fl32(x + c) for the fp16 value x in the low (hi = 0) or high half of `pair`: one
// mixed-precision FMA x * 1.0 + c, which rounds once, reading the half in place.
__device__ __forceinline__ float sub_half(uint32_t pair, int hi, float c) {
  float d;
  if (hi)
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(pair), "v"(c));
  else
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(pair), "v"(c));
  return d;
}

template <int LPG>
struct GroupQ {
  static_assert(LPG == 1 || LPG == 4 || LPG == 8, "1, 4 or 8 lanes per group");
  static constexpr int E = 64 / LPG;
  static constexpr int W = E / 8;     // 8-element vectors (and packed code words) per lane

  // x: this lane's E elements.  Returns the packed codes of those elements (E/2
  // bytes: E = 16 -> 8 bytes, E = 8 -> 4 bytes; code i of a word in bits 4i..4i+3)
  // in `packed` and the (offset, scale) pair as one 32-bit word.
  __device__ __forceinline__ static uint32_t run(const f16x8 (&x)[W], uint32_t (&packed)[W]) {
#pragma clang fp contract(off)
    // Group minimum and maximum on packed halves (fp16 comparisons are exact).  The
    // pair (min, -max) travels as one word through the cross-lane steps, where one
    // packed minimum updates both.
    f16x2 lo = __builtin_elementwise_minimum((f16x2){x[0][0], x[0][1]}, (f16x2){x[0][2], x[0][3]});
    f16x2 hi = __builtin_elementwise_maximum((f16x2){x[0][0], x[0][1]}, (f16x2){x[0][2], x[0][3]});
#pragma unroll
    for (int v = 0; v < W; ++v)
#pragma unroll
      for (int p = (v == 0 ? 2 : 0); p < 4; ++p) {
        const f16x2 e = (f16x2){x[v][2 * p], x[v][2 * p + 1]};
        lo = __builtin_elementwise_minimum(lo, e);
        hi = __builtin_elementwise_maximum(hi, e);
      }
    f16x2 mm = (f16x2){__builtin_elementwise_minimum(lo.x, lo.y),
                       -__builtin_elementwise_maximum(hi.x, hi.y)};
    if constexpr (LPG >= 4) {
      mm = __builtin_elementwise_minimum(mm, h2_from_u32(dpp_u32<0xB1>(u32_from_h2(mm))));
      mm = __builtin_elementwise_minimum(mm, h2_from_u32(dpp_u32<0x4E>(u32_from_h2(mm))));
    }
    if constexpr (LPG == 8)
      mm = __builtin_elementwise_minimum(mm, h2_from_u32(dpp_u32<0x141>(u32_from_h2(mm))));
    const float mn = (float)mm.x, mx = -(float)mm.y;

    const bool constant = (mx == mn);
    const float r = mx - mn;
    f16 s16 = (f16)(r / 15.0f);
    if (constant) s16 = (f16)0.0f;
    else if (s16 == (f16)0.0f) s16 = h_from_bits(0x0001);  // 2^-24
    const float sf = (float)s16;
    const float inv = constant ? 0.0f : 1.0f / sf;
    const float nmn = -mn;

    // t = fl32(fl32(x - min) * inv) lies in [0, 15.008] whenever the step is a normal
    // fp16 (its rounding error is below 2^-11), so the clamp is needed only for a
    // subnormal step.  v_cvt_pk_u8_f32 rounds to nearest even (checked on the chip
    // over every tie in [0, 16)) and drops rne(t) into one byte of a word: even codes
    // into the bytes of `lo`, odd codes into those of `hi`, and lo | hi << 4 is the
    // packed word (code i in bits 4i .. 4i + 3).
    const bool tiny = bits_from_h(s16) != 0 && (bits_from_h(s16) & 0x7C00) == 0;
    float t[E];
#pragma unroll
    for (int v = 0; v < W; ++v) {
      const u32x4 h = __builtin_bit_cast(u32x4, x[v]);
#pragma unroll
      for (int i = 0; i < 8; ++i) t[8 * v + i] = sub_half(h[i / 2], i % 2, nmn) * inv;
    }
    if (__builtin_amdgcn_ballot_w64(tiny)) {
#pragma unroll
      for (int i = 0; i < E; ++i) t[i] = fminf(t[i], 15.0f);
    }
#pragma unroll
    for (int v = 0; v < W; ++v) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        lo = __builtin_amdgcn_cvt_pk_u8_f32(t[8 * v + 2 * k], k, lo);
        hi = __builtin_amdgcn_cvt_pk_u8_f32(t[8 * v + 2 * k + 1], k, hi);
      }
      packed[v] = lo | (hi << 4);
    }
    const f16 off = (f16)(mn == 0.0f ? 0.0f : mn);
    return (uint32_t)bits_from_h(off) | ((uint32_t)bits_from_h(s16) << 16);
  }
};

}  // namespace flexq
