// Device-side group quantizer shared by the standalone quantize kernel, the prefill
// attention's KV store and the decode attention's append.
//
// A 64-element group is held by LPG consecutive lanes (LPG = 4 or 8), each lane
// holding E = 64 / LPG consecutive elements.  Arithmetic follows the compression
// step of the FlexGen walkthrough, section 6.3 (4 bits, group 64, asymmetric
// min/max), in fp32 with a fixed sequence so that codes are reproducible:
//   step   = fp16(fl32(max - min) / 15)   (0 if max == min; 2^-24 if it underflows)
//   code   = clamp(rne(fl32(x - min) * fl32(1 / step)), 0, 15)
//   offset = min (a zero minimum stored as +0)
#pragma once

#include "common.h"

namespace flexq {

template <int LPG>
struct GroupQ {
  static_assert(LPG == 4 || LPG == 8, "4 or 8 lanes per group");
  static constexpr int E = 64 / LPG;

  // x: this lane's E elements (fp16 values, exact in fp32).  Returns the packed
  // codes of those elements (E/2 bytes: E=16 -> 8 bytes, E=8 -> 4 bytes) in
  // `packed` and the (offset, scale) pair as one 32-bit word.
  __device__ __forceinline__ static uint32_t run(const float (&x)[E], uint32_t (&packed)[E / 8]) {
#pragma clang fp contract(off)
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < E; ++i) {
      mn = fminf(mn, x[i]);
      mx = fmaxf(mx, x[i]);
    }
    mn = fminf(mn, dpp_f32<0xB1>(mn));
    mx = fmaxf(mx, dpp_f32<0xB1>(mx));
    mn = fminf(mn, dpp_f32<0x4E>(mn));
    mx = fmaxf(mx, dpp_f32<0x4E>(mx));
    if constexpr (LPG == 8) {
      mn = fminf(mn, dpp_f32<0x141>(mn));
      mx = fmaxf(mx, dpp_f32<0x141>(mx));
    }
    const bool constant = (mx == mn);
    const float r = mx - mn;
    f16 s16 = (f16)(r / 15.0f);
    if (constant) s16 = (f16)0.0f;
    else if (s16 == (f16)0.0f) s16 = h_from_bits(0x0001);  // 2^-24
    const float sf = (float)s16;
    const float inv = constant ? 0.0f : 1.0f / sf;
#pragma unroll
    for (int w = 0; w < E / 8; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float t = (x[8 * w + i] - mn) * inv;
        t = fminf(fmaxf(t, 0.0f), 15.0f);
        const uint32_t c = (uint32_t)__builtin_rintf(t);
        word |= c << (4 * i);
      }
      packed[w] = word;
    }
    const f16 off = (f16)(mn == 0.0f ? 0.0f : mn);
    return (uint32_t)bits_from_h(off) | ((uint32_t)bits_from_h(s16) << 16);
  }
};

}  // namespace flexq
