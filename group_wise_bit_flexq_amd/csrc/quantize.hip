// Standalone group-wise 4-bit quantizer (`compress`) and weight dequantizer
// (`decompress`), FlexGen walkthrough section 6.3.
//
// Layout: groups are 64 consecutive elements of the innermost dimension, so the
// input is treated as a flat array of groups.  Each group is handled by 4 lanes
// holding 16 consecutive fp16 elements (32 B) each; a 256-thread block covers 64
// groups = 8 KiB of input.  A wave writes 512 B of codes contiguously (8 B per
// lane) and 16 parameter words.  HBM-bound: 2 B read + 0.5625 B written per element.
#include "quant_dev.h"

namespace flexq {

constexpr int kQLanes = 4;                     // lanes per group
constexpr int kQThreads = 256;
constexpr int kQGroupsPerBlock = kQThreads / kQLanes;

// WEIGHT = false: codes and params in row-major group order.  WEIGHT = true: the 4-bit
// weight layout (blocks of 128 rows, k-tile major, see w4_code_off; codes of a word in
// the order of w4_word_from_codes); ngroups then counts the rows padded to a multiple
// of 128, and the groups of pad rows are stored as zeros.
template <bool WEIGHT>
__global__ __launch_bounds__(kQThreads) void quantize_kernel(const uint4* __restrict__ x,
                                                             uint2* __restrict__ codes,
                                                             uint32_t* __restrict__ params,
                                                             int64_t ngroups, int64_t nreal,
                                                             int64_t KT) {
  const int64_t g = (int64_t)blockIdx.x * kQGroupsPerBlock + threadIdx.x / kQLanes;
  const int part = threadIdx.x % kQLanes;
  // all lanes of a wave take part in the cross-lane reduction; lanes past the end
  // work on a copy of the last group and store nothing
  const int64_t gl = g < nreal ? g : nreal - 1;
  const uint4 a = x[gl * 8 + part * 2];
  const uint4 b = x[gl * 8 + part * 2 + 1];
  const f16x8 v[2] = {__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b)};
  uint32_t packed[2];
  uint32_t p = GroupQ<kQLanes>::run(v, packed);
  if (g < ngroups) {
    if constexpr (WEIGHT) {
      if (g >= nreal) packed[0] = packed[1] = p = 0;
      const int64_t row = g / KT, kt = g - row * KT;
      codes[w4_code_off(row, kt, KT) / 8 + part] =
          make_uint2(w4_word_from_codes(packed[0]), w4_word_from_codes(packed[1]));
      if (part == 0) params[w4_param_idx(row, kt, KT)] = p;
    } else {
      codes[g * 4 + part] = make_uint2(packed[0], packed[1]);
      if (part == 0) params[g] = p;
    }
  }
}

// out = fp16(c * s + m), one rounding; each thread expands 16 codes (8 B).
__global__ __launch_bounds__(256) void dequantize_kernel(const uint2* __restrict__ codes,
                                                         const uint32_t* __restrict__ params,
                                                         uint4* __restrict__ out, int64_t nchunks) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 16-element chunk
  if (i >= nchunks) return;
  const uint2 c = codes[i];
  const uint32_t p = params[i / 4];
  const f16x2 m2 = h2_from_u32((p & 0xFFFFu) * 0x10001u);
  const f16x2 s2 = h2_from_u32((p >> 16) * 0x10001u);
  f16x2 pr[8];
  codes_to_pairs(c.x, pr);
  codes_to_pairs(c.y, pr + 4);
  uint32_t o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = u32_from_h2(dequant_pair(pr[k], s2, m2));
  out[2 * i] = make_uint4(o[0], o[1], o[2], o[3]);
  out[2 * i + 1] = make_uint4(o[4], o[5], o[6], o[7]);
}

}  // namespace flexq

using namespace flexq;

extern "C" const char* flexq_status_string(int s) {
  switch (s) {
    case FLEXQ_OK: return "ok";
    case FLEXQ_ERR_INVALID: return "invalid argument";
    case FLEXQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case FLEXQ_ERR_DEVICE: return "device/launch error";
    default: return "unknown status";
  }
}

static int quantize_entry(bool weight, const uint16_t* x, int64_t rows, int64_t cols,
                          flexq_qconfig cfg, uint8_t* codes, uint16_t* params, hipStream_t stream) {
  if (cfg.num_bits != 4 || cfg.group_size != 64 || cfg.symmetric != 0) return FLEXQ_ERR_UNSUPPORTED;
  if (rows < 0 || cols <= 0 || cols % 64 != 0) return FLEXQ_ERR_INVALID;
  if (rows == 0) return FLEXQ_OK;
  if (!x || !codes || !params) return FLEXQ_ERR_INVALID;
  if (((uintptr_t)x & 15) || ((uintptr_t)codes & 7) || ((uintptr_t)params & 3)) return FLEXQ_ERR_INVALID;
  const int64_t KT = cols / 64;
  const int64_t nreal = rows * KT;
  const int64_t ngroups = weight ? (rows + kW4BlockRows - 1) / kW4BlockRows * kW4BlockRows * KT : nreal;
  const int64_t blocks = (ngroups + kQGroupsPerBlock - 1) / kQGroupsPerBlock;
  if (blocks > 0x7FFFFFFF) return FLEXQ_ERR_UNSUPPORTED;
  if (weight)
    hipLaunchKernelGGL(quantize_kernel<true>, dim3((unsigned)blocks), dim3(kQThreads), 0, stream,
                       (const uint4*)x, (uint2*)codes, (uint32_t*)params, ngroups, nreal, KT);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, dim3((unsigned)blocks), dim3(kQThreads), 0, stream,
                       (const uint4*)x, (uint2*)codes, (uint32_t*)params, ngroups, nreal, KT);
  FLEXQ_LAUNCH_CHECK();
  return FLEXQ_OK;
}

extern "C" int flexq_quantize(const uint16_t* x, int64_t rows, int64_t cols, flexq_qconfig cfg,
                              uint8_t* codes, uint16_t* params, hipStream_t stream) {
  return quantize_entry(false, x, rows, cols, cfg, codes, params, stream);
}

extern "C" int flexq_quantize_w4(const uint16_t* x, int64_t rows, int64_t cols, flexq_qconfig cfg,
                                 uint8_t* codes, uint16_t* params, hipStream_t stream) {
  return quantize_entry(true, x, rows, cols, cfg, codes, params, stream);
}

extern "C" int flexq_dequantize(const uint8_t* codes, const uint16_t* params, int64_t rows,
                                int64_t cols, uint16_t* out, hipStream_t stream) {
  if (rows < 0 || cols <= 0 || cols % 64 != 0) return FLEXQ_ERR_INVALID;
  if (rows == 0) return FLEXQ_OK;
  if (!codes || !params || !out) return FLEXQ_ERR_INVALID;
  if (((uintptr_t)out & 15) || ((uintptr_t)codes & 7) || ((uintptr_t)params & 3)) return FLEXQ_ERR_INVALID;
  const int64_t nchunks = rows * cols / 16;
  const int64_t blocks = (nchunks + 255) / 256;
  if (blocks > 0x7FFFFFFF) return FLEXQ_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint2*)codes, (const uint32_t*)params, (uint4*)out, nchunks);
  FLEXQ_LAUNCH_CHECK();
  return FLEXQ_OK;
}
