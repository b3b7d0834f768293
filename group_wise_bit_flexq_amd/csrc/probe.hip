// Measurement aid: the matrix cores' sustained fp16 rate on this chip, for the
// roofline reported next to the GEMMs.  Not part of the decoder path.
//
// Every wave streams v_mfma_f32_32x32x16_f16 on four independent accumulators (no
// dependence between consecutive MFMAs), two waves per SIMD.  The operands are
//   mode 0: constant (every fp16 operand 1.0);
//   mode 1: fixed pseudo-random fp16 values in +-[0.5, 1), drawn once per lane;
//   mode 2: the mode-1 values with mantissa bits flipped every iteration (one XOR per
//           operand register per four MFMAs), as real GEMM operands change.
// The chip's power management lowers the clock as operand bits toggle, so the three
// modes bound what a GEMM on real data can reach.
#include "common.h"

namespace flexq {

template <int MODE>
__global__ __launch_bounds__(256, 2) void mfma_probe_kernel(int iters, float* __restrict__ out) {
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t h = gid * 0x9E3779B9u + 0x7F4A7C15u;
  u32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (MODE == 0) {
      a[i] = 0x3C003C00u;   // (1.0, 1.0)
      b[i] = 0x3C003C00u;
    } else {
      // fp16 in +-[0.5, 1): exponent 14, random sign and mantissa
      h ^= h << 13; h ^= h >> 17; h ^= h << 5;
      a[i] = (h & 0x83FF83FFu) | 0x38003800u;
      h ^= h << 13; h ^= h >> 17; h ^= h << 5;
      b[i] = (h & 0x83FF83FFu) | 0x38003800u;
    }
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const u32x4 flip = {0x02AA0155u, 0x015502AAu, 0x00FF0300u, 0x030000FFu};
  for (int it = 0; it < iters; ++it) {
    const f16x8 av = __builtin_bit_cast(f16x8, a), bv = __builtin_bit_cast(f16x8, b);
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, c3, 0, 0, 0);
    if constexpr (MODE == 2) {
      a ^= flip;   // mantissa bits only: values stay in +-[0.5, 1)
      b ^= flip.yxwz;
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[gid] = s;
}

}  // namespace flexq

using namespace flexq;

extern "C" int flexq_probe_mfma(int32_t mode, int32_t blocks, int32_t iters, float* out,
                                hipStream_t stream) {
  if (mode < 0 || mode > 2 || blocks <= 0 || iters <= 0 || !out) return FLEXQ_ERR_INVALID;
  if (mode == 0)
    hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3(blocks), dim3(256), 0, stream, iters, out);
  else if (mode == 1)
    hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3(blocks), dim3(256), 0, stream, iters, out);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<2>, dim3(blocks), dim3(256), 0, stream, iters, out);
  FLEXQ_LAUNCH_CHECK();
  return FLEXQ_OK;
}
