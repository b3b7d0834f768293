// Group-wise quantization with a general compression config: num_bits 2..8,
// asymmetric or symmetric, any group size, any grouped axis, ragged lengths
// (FlexGen walkthrough section 6.3 names the config's fields num_bits, group_size,
// group_dim and symmetric; the hub page's section on its core principles mentions
// int3 and int4).
//
// The tensor is seen as [outer][n][inner] with groups of `group_size` consecutive
// positions along n (the grouped axis; inner = 1 when it is the innermost one).  The
// last group of a ragged n is zero-padded, and the padding is quantized with its
// group like any element.  Per group, in fp32 with contraction off:
//   asymmetric: step = fp16((max - min) / (2^b - 1)), code = clamp(rne((x - min) *
//               (1 / step)), 0, 2^b - 1), offset = min (+0 for a zero minimum);
//   symmetric:  B = 2^(b-1) - 1, step = fp16(max|x| / B), code = clamp(rne(x *
//               (1 / step)), -B, B) + 2^(b-1), offset = +0;
//   a constant (asymmetric) or all-zero (symmetric) group gets step 0; a step that
//   underflows fp16 becomes 2^-24.
// The b-bit codes of a group are concatenated least significant bit first into
// group_size * b / 8 bytes, which lie along n in the packed tensor
// [outer][num_groups * group_size * b / 8][inner]; params are
// [outer][num_groups][inner] (offset, step) fp16 pairs.
//
// Grouped axis innermost and group_size 16, 32, 64 or 128: L = group_size / 16 lanes
// per group, 16 consecutive elements (two 16-B loads) per lane, the group statistics
// reduced across the L lanes with DPP moves; a lane's 16 codes are 2b bytes, stored
// as b 16-bit words.  Otherwise one thread per (outer, group, inner) reads its group
// with strided loads, coalesced across the consecutive inner indices of a wave, and
// keeps it in registers for group sizes 16, 32 and 64 (else it reads it twice); then a
// thread takes 4 (groups of 16 or 32) or 2 (groups of 64) consecutive inner positions.
#include "quant_dev.h"

namespace flexq {


struct QxShape {
  int64_t outer, n, inner;
  int ng, gsize, bits, gbytes;
};

// step and 1 / step of a group from its statistics (min and max, or 0 and max|x|)
__device__ __forceinline__ void qx_step(bool sym, int bits, float lo, float hi, f16& step,
                                        float& inv, bool& constant) {
#pragma clang fp contract(off)
  const int qmax = sym ? (1 << (bits - 1)) - 1 : (1 << bits) - 1;
  constant = sym ? (hi == 0.0f) : (hi == lo);
  const float r = sym ? hi : hi - lo;
  f16 s = (f16)(r / (float)qmax);
  if (constant) s = (f16)0.0f;
  else if (s == (f16)0.0f) s = h_from_bits(0x0001);   // 2^-24
  step = s;
  inv = constant ? 0.0f : 1.0f / (float)s;
}

__device__ __forceinline__ uint32_t qx_code(bool sym, int bits, float x, float mn, float inv) {
#pragma clang fp contract(off)
  if (sym) {
    const float qm = (float)((1 << (bits - 1)) - 1);
    const float t = fminf(fmaxf(x * inv, -qm), qm);
    return (uint32_t)((int)__builtin_rintf(t) + (1 << (bits - 1)));
  }
  const float t = fminf(fmaxf((x - mn) * inv, 0.0f), (float)((1 << bits) - 1));
  return (uint32_t)__builtin_rintf(t);
}

// Appends a b-bit code to the bit accumulator and writes out every full byte (bytes
// along n, `stride` apart).
struct QxPacker {
  uint64_t acc = 0;
  int nbits = 0;
  int64_t byte = 0;
  __device__ __forceinline__ void put(uint32_t c, int bits, uint8_t* __restrict__ dst,
                                      int64_t stride) {
    acc |= (uint64_t)c << nbits;
    nbits += bits;
    while (nbits >= 8) {
      dst[byte * stride] = (uint8_t)(acc & 0xFFu);
      acc >>= 8;
      nbits -= 8;
      ++byte;
    }
  }
};

// min and max (or 0 and max|x|) over the L lanes of a group (aligned lane groups)
template <int L>
__device__ __forceinline__ void qx_reduce(float& lo, float& hi) {
  if constexpr (L >= 2) {
    lo = fminf(lo, dpp_f32<0xB1>(lo));
    hi = fmaxf(hi, dpp_f32<0xB1>(hi));
  }
  if constexpr (L >= 4) {
    lo = fminf(lo, dpp_f32<0x4E>(lo));
    hi = fmaxf(hi, dpp_f32<0x4E>(hi));
  }
  if constexpr (L >= 8) {
    lo = fminf(lo, dpp_f32<0x141>(lo));
    hi = fmaxf(hi, dpp_f32<0x141>(hi));
  }
}

// Grouped axis innermost (inner == 1), n a multiple of 8, x 16-B aligned:
// group_size = 16 L, lanes 16 part .. 16 part + 15 of a group in lane part.
template <bool SYM, int L>
__global__ __launch_bounds__(256) void quantize_ex_lanes_kernel(const f16* __restrict__ x,
                                                                uint8_t* __restrict__ codes,
                                                                uint32_t* __restrict__ params,
                                                                QxShape sh) {
#pragma clang fp contract(off)
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t ngroups = sh.outer * sh.ng;
  const int part = (int)(t % L);
  const int64_t gflat = t / L;
  // every lane of a wave takes part in the DPP reduction: lanes past the end work on
  // the last group and store nothing
  const int64_t gl = gflat < ngroups ? gflat : ngroups - 1;
  const int64_t o = gl / sh.ng;
  const int g = (int)(gl - o * sh.ng);
  const int64_t k0 = (int64_t)g * (16 * L) + 16 * part;
  const f16* xs = x + o * sh.n;
  f16x8 v[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t k = k0 + 8 * q;
    if (k + 8 <= sh.n) {
      v[q] = *(const f16x8*)(xs + k);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[q][e] = (f16)0.0f;   // n % 8 == 0: the whole chunk is padding
    }
  }
  float lo = SYM ? 0.0f : INFINITY, hi = SYM ? 0.0f : -INFINITY;
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = (float)v[q][e];
      if (SYM) hi = fmaxf(hi, fabsf(f));
      else { lo = fminf(lo, f); hi = fmaxf(hi, f); }
    }
  qx_reduce<L>(lo, hi);
  f16 step;
  float inv;
  bool constant;
  qx_step(SYM, sh.bits, lo, hi, step, inv, constant);
  if (gflat >= ngroups) return;
  // 16 codes = 2b bytes = b 16-bit words at byte 2 b part of the group's gb bytes
  uint16_t* dst = (uint16_t*)(codes + gl * sh.gbytes) + sh.bits * part;
  uint64_t acc = 0;
  int nbits = 0, w = 0;
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc |= (uint64_t)qx_code(SYM, sh.bits, (float)v[q][e], lo, inv) << nbits;
      nbits += sh.bits;
      if (nbits >= 16) {
        dst[w++] = (uint16_t)(acc & 0xFFFFu);
        acc >>= 16;
        nbits -= 16;
      }
    }
  if (part == 0) {
    const f16 off = SYM ? (f16)0.0f : (f16)(lo == 0.0f ? 0.0f : lo);
    params[gl] = (uint32_t)bits_from_h(off) | ((uint32_t)bits_from_h(step) << 16);
  }
}

// Any layout: one thread per (outer, group, inner), elements k * inner apart.  GS > 0:
// the group size is GS and the thread keeps the group in registers (one read);
// GS == 0: any group size, the group is read twice.
template <bool SYM, int GS>
__global__ __launch_bounds__(256) void quantize_ex_kernel(const f16* __restrict__ x,
                                                          uint8_t* __restrict__ codes,
                                                          uint32_t* __restrict__ params,
                                                          QxShape sh) {
#pragma clang fp contract(off)
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = sh.outer * sh.ng * sh.inner;
  if (t >= total) return;
  const int64_t i = t % sh.inner;
  const int64_t rest = t / sh.inner;
  const int g = (int)(rest % sh.ng);
  const int64_t o = rest / sh.ng;
  const int gsize = GS > 0 ? GS : sh.gsize;
  const int64_t k0 = (int64_t)g * gsize;                    // first position along n
  const f16* xs = x + o * sh.n * sh.inner + i;              // position k at xs[k * inner]
  uint8_t* cdst = codes + (o * sh.ng * sh.gbytes + (int64_t)g * sh.gbytes) * sh.inner + i;
  float lo = SYM ? 0.0f : INFINITY, hi = SYM ? 0.0f : -INFINITY;
  f16 step;
  float inv;
  bool constant;
  QxPacker pk;
  if constexpr (GS > 0) {
    f16 v[GS];
#pragma unroll
    for (int e = 0; e < GS; ++e) v[e] = k0 + e < sh.n ? xs[(k0 + e) * sh.inner] : (f16)0.0f;
#pragma unroll
    for (int e = 0; e < GS; ++e) {
      const float f = (float)v[e];
      if (SYM) hi = fmaxf(hi, fabsf(f));
      else { lo = fminf(lo, f); hi = fmaxf(hi, f); }
    }
    qx_step(SYM, sh.bits, lo, hi, step, inv, constant);
#pragma unroll
    for (int e = 0; e < GS; ++e) pk.put(qx_code(SYM, sh.bits, (float)v[e], lo, inv), sh.bits, cdst, sh.inner);
  } else {
    for (int e = 0; e < gsize; ++e) {
      const int64_t k = k0 + e;
      const float f = k < sh.n ? (float)xs[k * sh.inner] : 0.0f;
      if (SYM) hi = fmaxf(hi, fabsf(f));
      else { lo = fminf(lo, f); hi = fmaxf(hi, f); }
    }
    qx_step(SYM, sh.bits, lo, hi, step, inv, constant);
    for (int e = 0; e < gsize; ++e) {
      const int64_t k = k0 + e;
      const float f = k < sh.n ? (float)xs[k * sh.inner] : 0.0f;
      pk.put(qx_code(SYM, sh.bits, f, lo, inv), sh.bits, cdst, sh.inner);
    }
  }
  const f16 off = SYM ? (f16)0.0f : (f16)(lo == 0.0f ? 0.0f : lo);
  params[(o * sh.ng + g) * sh.inner + i] = (uint32_t)bits_from_h(off) | ((uint32_t)bits_from_h(step) << 16);
}

// Strided layout, V = 2 or 4 consecutive inner positions per thread (inner % V == 0;
// x 2V-B, codes and params V-B and 4-B aligned), group size GS kept in registers: 2V-B
// loads, the V groups quantized in lockstep, their code bytes (equal bit positions)
// stored as one V-byte word.
template <int V> struct QxVec;
template <> struct QxVec<2> { typedef f16x2 h; typedef uint16_t w; };
template <> struct QxVec<4> { typedef f16x4 h; typedef uint32_t w; };

template <bool SYM, int GS, int V>
__global__ __launch_bounds__(256) void quantize_ex_vec_kernel(const f16* __restrict__ x,
                                                              uint8_t* __restrict__ codes,
                                                              uint32_t* __restrict__ params,
                                                              QxShape sh) {
#pragma clang fp contract(off)
  typedef typename QxVec<V>::h hv;
  typedef typename QxVec<V>::w wv;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t inv_ = sh.inner / V;
  const int64_t total = sh.outer * sh.ng * inv_;
  if (t >= total) return;
  const int64_t i = V * (t % inv_);
  const int64_t rest = t / inv_;
  const int g = (int)(rest % sh.ng);
  const int64_t o = rest / sh.ng;
  const int64_t k0 = (int64_t)g * GS;
  const f16* xs = x + o * sh.n * sh.inner + i;
  hv v[GS];
#pragma unroll
  for (int e = 0; e < GS; ++e) {
    if (k0 + e < sh.n) v[e] = *(const hv*)(xs + (k0 + e) * sh.inner);
    else
#pragma unroll
      for (int c = 0; c < V; ++c) v[e][c] = (f16)0.0f;
  }
  float lo[V], hi[V], inv[V];
  f16 step[V];
#pragma unroll
  for (int c = 0; c < V; ++c) {
    lo[c] = SYM ? 0.0f : INFINITY;
    hi[c] = SYM ? 0.0f : -INFINITY;
  }
#pragma unroll
  for (int e = 0; e < GS; ++e)
#pragma unroll
    for (int c = 0; c < V; ++c) {
      const float f = (float)v[e][c];
      if (SYM) hi[c] = fmaxf(hi[c], fabsf(f));
      else { lo[c] = fminf(lo[c], f); hi[c] = fmaxf(hi[c], f); }
    }
#pragma unroll
  for (int c = 0; c < V; ++c) {
    bool constant;
    qx_step(SYM, sh.bits, lo[c], hi[c], step[c], inv[c], constant);
  }
  wv* cdst = (wv*)(codes + (o * sh.ng * sh.gbytes + (int64_t)g * sh.gbytes) * sh.inner + i);
  const int64_t wstride = sh.inner / V;        // words between consecutive code bytes
  uint64_t acc[V];
#pragma unroll
  for (int c = 0; c < V; ++c) acc[c] = 0;
  int nbits = 0;
  int64_t byte = 0;
#pragma unroll
  for (int e = 0; e < GS; ++e) {
#pragma unroll
    for (int c = 0; c < V; ++c) acc[c] |= (uint64_t)qx_code(SYM, sh.bits, (float)v[e][c], lo[c], inv[c]) << nbits;
    nbits += sh.bits;
    while (nbits >= 8) {
      uint32_t wd = 0;
#pragma unroll
      for (int c = 0; c < V; ++c) {
        wd |= (uint32_t)(acc[c] & 0xFFu) << (8 * c);
        acc[c] >>= 8;
      }
      cdst[byte * wstride] = (wv)wd;
      nbits -= 8;
      ++byte;
    }
  }
  uint32_t* pdst = params + (o * sh.ng + g) * sh.inner + i;
#pragma unroll
  for (int c = 0; c < V; ++c) {
    const f16 off = SYM ? (f16)0.0f : (f16)(lo[c] == 0.0f ? 0.0f : lo[c]);
    pdst[c] = (uint32_t)bits_from_h(off) | ((uint32_t)bits_from_h(step[c]) << 16);
  }
}

// fp16 values of the codes: fp16(code * step + offset) or fp16((code - 2^(b-1)) * step),
// each one rounding of the exact value (fp16 FMA of exact operands: |code| <= 255).
template <bool SYM>
__global__ __launch_bounds__(256) void dequantize_ex_kernel(const uint8_t* __restrict__ codes,
                                                            const uint32_t* __restrict__ params,
                                                            f16* __restrict__ out, QxShape sh) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = sh.outer * sh.ng * sh.inner;
  if (t >= total) return;
  const int64_t i = t % sh.inner;
  const int64_t rest = t / sh.inner;
  const int g = (int)(rest % sh.ng);
  const int64_t o = rest / sh.ng;
  const uint32_t p = params[(o * sh.ng + g) * sh.inner + i];
  const f16 m = h_from_bits((uint16_t)(p & 0xFFFFu));
  const f16 s = h_from_bits((uint16_t)(p >> 16));
  const uint8_t* csrc = codes + (o * sh.ng * sh.gbytes + (int64_t)g * sh.gbytes) * sh.inner + i;
  f16* dst = out + o * sh.n * sh.inner + i;
  uint64_t acc = 0;
  int nbits = 0;
  int64_t byte = 0;
  const uint32_t mask = (1u << sh.bits) - 1u;
  for (int e = 0; e < sh.gsize; ++e) {
    while (nbits < sh.bits) {
      acc |= (uint64_t)csrc[byte * sh.inner] << nbits;
      nbits += 8;
      ++byte;
    }
    const uint32_t c = (uint32_t)acc & mask;
    acc >>= sh.bits;
    nbits -= sh.bits;
    const int64_t k = (int64_t)g * sh.gsize + e;
    if (k < sh.n) {
      f16 v;
      if (SYM) v = __builtin_fmaf16((f16)(float)((int)c - (1 << (sh.bits - 1))), s, (f16)0.0f);
      else v = __builtin_fmaf16((f16)(float)c, s, m);
      dst[k * sh.inner] = v;
    }
  }
}

static int qx_shape(int64_t outer, int64_t n, int64_t inner, flexq_qconfig cfg, QxShape& sh) {
  if (cfg.num_bits < 2 || cfg.num_bits > 8 || cfg.group_size < 1 || cfg.group_size > 4096 ||
      (cfg.symmetric != 0 && cfg.symmetric != 1) || (cfg.group_size * cfg.num_bits) % 8)
    return FLEXQ_ERR_UNSUPPORTED;
  if (outer < 0 || n < 0 || inner < 0) return FLEXQ_ERR_INVALID;
  sh.outer = outer;
  sh.n = n;
  sh.inner = inner;
  sh.gsize = cfg.group_size;
  sh.bits = cfg.num_bits;
  sh.gbytes = cfg.group_size * cfg.num_bits / 8;
  const int64_t ng = (n + cfg.group_size - 1) / cfg.group_size;
  if (ng > 0x7FFFFFFF) return FLEXQ_ERR_UNSUPPORTED;
  sh.ng = (int)ng;
  return FLEXQ_OK;
}

}  // namespace flexq

using namespace flexq;

extern "C" int flexq_quantize_ex(const uint16_t* x, int64_t outer, int64_t n, int64_t inner,
                                 flexq_qconfig cfg, uint8_t* codes, uint16_t* params,
                                 hipStream_t stream) {
  QxShape sh;
  const int st = qx_shape(outer, n, inner, cfg, sh);
  if (st != FLEXQ_OK) return st;
  const int64_t total = sh.outer * sh.ng * sh.inner;
  if (total == 0) return FLEXQ_OK;
  if (!x || !codes || !params || ((uintptr_t)params & 3) || ((uintptr_t)x & 1))
    return FLEXQ_ERR_INVALID;
  const int L = sh.gsize / 16;
  const bool lanes = sh.inner == 1 && sh.gsize % 16 == 0 && (L == 1 || L == 2 || L == 4 || L == 8) &&
                     ((uintptr_t)x & 15) == 0 && sh.n % 8 == 0 && ((uintptr_t)codes & 1) == 0;
  // strided groups of 16 / 32 take 4 inner positions per thread, of 64 take 2
  const int V = sh.gsize == 64 ? 2 : 4;
  const bool vec = !lanes && (sh.gsize == 16 || sh.gsize == 32 || sh.gsize == 64) &&
                   sh.inner % V == 0 && ((uintptr_t)x & (2 * V - 1)) == 0 &&
                   ((uintptr_t)codes & (V - 1)) == 0;
  const int64_t threads = lanes ? sh.outer * sh.ng * L : vec ? total / V : total;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7FFFFFFF) return FLEXQ_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)blocks), block(256);
  const f16* xh = (const f16*)x;
  uint32_t* pw = (uint32_t*)params;
#define QX_LANES(SYM_, L_) \
  hipLaunchKernelGGL((quantize_ex_lanes_kernel<SYM_, L_>), grid, block, 0, stream, xh, codes, pw, sh)
  if (lanes) {
    if (cfg.symmetric) {
      if (L == 1) QX_LANES(true, 1); else if (L == 2) QX_LANES(true, 2);
      else if (L == 4) QX_LANES(true, 4); else QX_LANES(true, 8);
    } else {
      if (L == 1) QX_LANES(false, 1); else if (L == 2) QX_LANES(false, 2);
      else if (L == 4) QX_LANES(false, 4); else QX_LANES(false, 8);
    }
  } else if (vec) {
#define QX_VEC(SYM_, GS_, V_) \
  hipLaunchKernelGGL((quantize_ex_vec_kernel<SYM_, GS_, V_>), grid, block, 0, stream, xh, codes, pw, sh)
    if (cfg.symmetric) {
      if (sh.gsize == 16) QX_VEC(true, 16, 4); else if (sh.gsize == 32) QX_VEC(true, 32, 4);
      else QX_VEC(true, 64, 2);
    } else {
      if (sh.gsize == 16) QX_VEC(false, 16, 4); else if (sh.gsize == 32) QX_VEC(false, 32, 4);
      else QX_VEC(false, 64, 2);
    }
#undef QX_VEC
  } else {
#define QX_STRIDED(SYM_, GS_) \
  hipLaunchKernelGGL((quantize_ex_kernel<SYM_, GS_>), grid, block, 0, stream, xh, codes, pw, sh)
    if (cfg.symmetric) {
      if (sh.gsize == 16) QX_STRIDED(true, 16); else if (sh.gsize == 32) QX_STRIDED(true, 32);
      else if (sh.gsize == 64) QX_STRIDED(true, 64); else QX_STRIDED(true, 0);
    } else {
      if (sh.gsize == 16) QX_STRIDED(false, 16); else if (sh.gsize == 32) QX_STRIDED(false, 32);
      else if (sh.gsize == 64) QX_STRIDED(false, 64); else QX_STRIDED(false, 0);
    }
#undef QX_STRIDED
  }
#undef QX_LANES
  FLEXQ_LAUNCH_CHECK();
  return FLEXQ_OK;
}

extern "C" int flexq_dequantize_ex(const uint8_t* codes, const uint16_t* params, int64_t outer,
                                   int64_t n, int64_t inner, flexq_qconfig cfg, uint16_t* out,
                                   hipStream_t stream) {
  QxShape sh;
  const int st = qx_shape(outer, n, inner, cfg, sh);
  if (st != FLEXQ_OK) return st;
  const int64_t total = sh.outer * sh.ng * sh.inner;
  if (total == 0) return FLEXQ_OK;
  if (!codes || !params || !out || ((uintptr_t)params & 3) || ((uintptr_t)out & 1))
    return FLEXQ_ERR_INVALID;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFF) return FLEXQ_ERR_UNSUPPORTED;
  if (cfg.symmetric)
    hipLaunchKernelGGL(dequantize_ex_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       codes, (const uint32_t*)params, (f16*)out, sh);
  else
    hipLaunchKernelGGL(dequantize_ex_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       codes, (const uint32_t*)params, (f16*)out, sh);
  FLEXQ_LAUNCH_CHECK();
  return FLEXQ_OK;
}
