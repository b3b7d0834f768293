// Row kernels around the GEMMs: LayerNorm, token + position embedding
// (`opt_input_embed`), greedy argmax over logits (`opt_output_embed`'s pick);
// source notes, section "Pytorch Backend".  All HBM-bound and small next to the
// GEMMs and attention.
#include "common.h"
#include "pick.h"

namespace flexq {

constexpr int kLnThreads = 256;
constexpr int kLnMaxChunks = 8;  // 8 x 256 x 8 = 16384 >= every hidden size here

// One work-group per row; the row stays in registers between the two passes.
__global__ __launch_bounds__(kLnThreads) void layernorm_kernel(const f16* __restrict__ x,
                                                               int64_t x_stride, int h,
                                                               const f16* __restrict__ g,
                                                               const f16* __restrict__ b,
                                                               f16* __restrict__ y) {
  __shared__ float red[8];
  const int64_t row = blockIdx.x;
  const f16* xr = x + row * x_stride;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = h / 8;
  f16x8 v[kLnMaxChunks];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kLnMaxChunks; ++i) {
    const int c = tid + i * kLnThreads;
    if (c < nch) {
      v[i] = *(const f16x8*)(xr + c * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += (float)v[i][e];
    }
  }
  s = wave_sum(s);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  const float mean = ((red[0] + red[1]) + (red[2] + red[3])) / (float)h;
  float q = 0.0f;
#pragma unroll
  for (int i = 0; i < kLnMaxChunks; ++i) {
    const int c = tid + i * kLnThreads;
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = (float)v[i][e] - mean;
        q += d * d;
      }
    }
  }
  q = wave_sum(q);
  if (lane == 0) red[4 + wave] = q;
  __syncthreads();
  const float var = ((red[4] + red[5]) + (red[6] + red[7])) / (float)h;
  const float rstd = 1.0f / sqrtf(var + 1e-5f);
  f16* yr = y + row * h;
#pragma unroll
  for (int i = 0; i < kLnMaxChunks; ++i) {
    const int c = tid + i * kLnThreads;
    if (c < nch) {
      const f16x8 gg = *(const f16x8*)(g + c * 8);
      const f16x8 bb = *(const f16x8*)(b + c * 8);
      f16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        o[e] = (f16)(((float)v[i][e] - mean) * rstd * (float)gg[e] + (float)bb[e]);
      *(f16x8*)(yr + c * 8) = o;
    }
  }
}

// out[m][k] = fp16(fp16(c * s + off) + pos[p + 2][k]) with p = pos_base + m % seq
// - pad[m / seq] (left padding; p >= 0).  One work-group per row, 16 elements per
// thread and step.
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tokens,
                                                    int pos_base, int seq,
                                                    const int32_t* __restrict__ pad, int h,
                                                    const uint2* __restrict__ codes,
                                                    const uint32_t* __restrict__ params,
                                                    const f16* __restrict__ pos, int pos_rows,
                                                    int vocab, f16* __restrict__ out) {
  const int64_t m = blockIdx.x;
  int tok = tokens[m];
  tok = tok < 0 ? 0 : (tok >= vocab ? vocab - 1 : tok);
  int p = pos_base + (int)(m % seq) - (pad ? pad[m / seq] : 0);
  p = (p < 0 ? 0 : p) + 2;
  p = p >= pos_rows ? pos_rows - 1 : p;
  const int KT = h / 64;
  for (int c = threadIdx.x; c < h / 16; c += blockDim.x) {
    // 16-element chunk c = bytes 8 (c % 4) .. +8 of k-tile c / 4 (4-bit weight layout)
    const uint2 cw = codes[w4_code_off(tok, c / 4, KT) / 8 + (c & 3)];
    const uint32_t prm = params[w4_param_idx(tok, c / 4, KT)];
    const f16x2 m2 = h2_from_u32((prm & 0xFFFFu) * 0x10001u);
    const f16x2 s2 = h2_from_u32((prm >> 16) * 0x10001u);
    f16x2 pr[8];
    w4_word_to_pairs(cw.x, pr);
    w4_word_to_pairs(cw.y, pr + 4);
    const f16x8* pp = (const f16x8*)(pos + (int64_t)p * h + c * 16);
    const f16x8 p0 = pp[0], p1 = pp[1];
    f16x8 o0, o1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f16x2 a = dequant_pair(pr[k], s2, m2);
      const f16x2 bb = dequant_pair(pr[4 + k], s2, m2);
      o0[2 * k] = (f16)((float)a.x + (float)p0[2 * k]);
      o0[2 * k + 1] = (f16)((float)a.y + (float)p0[2 * k + 1]);
      o1[2 * k] = (f16)((float)bb.x + (float)p1[2 * k]);
      o1[2 * k + 1] = (f16)((float)bb.y + (float)p1[2 * k + 1]);
    }
    f16x8* op = (f16x8*)(out + m * h + c * 16);
    op[0] = o0;
    op[1] = o1;
  }
}

__device__ __forceinline__ void better(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

__device__ __forceinline__ void better(double& v, int& i, double v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

// SplitMix64: output number c from state `seed` is mix(seed + (c + 1) * golden), with
// the published golden-ratio increment, mixing multipliers and shifts (64-bit
// wrap-around arithmetic).  `splitmix64_mix` takes the already-advanced state.
constexpr uint64_t kGolden64 = 0x9E3779B97F4A7C15ull;
__device__ __forceinline__ uint64_t splitmix64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Block-wide reduction of (value, index) pairs; the result is valid in thread 0.
template <int THREADS, typename T>
__device__ __forceinline__ void block_best(T& bv, int& bi) {
  __shared__ T sv[THREADS / 64];
  __shared__ int si[THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const T v2 = __shfl_xor(bv, o, 64);
    const int i2 = __shfl_xor(bi, o, 64);
    better(bv, bi, v2, i2);
  }
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (tid == 0)
    for (int w = 1; w < THREADS / 64; ++w) better(bv, bi, sv[w], si[w]);
}

// Next token of one row per work-group.  Greedy: the largest logit.  Sampling: the
// Gumbel-max draw argmax_n (logit_n / T - log(-log u_n)) in fp64, u_n from
// SplitMix64 output (step << 48 | sequence << 32 | n) mapped to ((z >> 12) + 1/2) 2^-52.
// Lowest index among equal maxima in both.  With a stop token, a row already
// stopped emits it again, and a row that emits it becomes stopped (`fresh`: the
// incoming flags are ignored, as for the first token of a sequence).
template <bool SAMPLE, int THREADS>
__global__ __launch_bounds__(THREADS) void pick_kernel(const float* __restrict__ logits, int64_t N,
                                                       uint64_t seed, double temperature,
                                                       uint32_t step, uint32_t m0, int32_t stop,
                                                       int32_t* __restrict__ stopped, int fresh,
                                                       int32_t* __restrict__ next) {
  const int m = blockIdx.x;
  if (stopped && !fresh && stopped[m]) {  // uniform over the work-group
    if (threadIdx.x == 0) next[m] = stop;
    return;
  }
  const float* r = logits + (int64_t)m * N;
  int bi = 0x7FFFFFFF;
  if constexpr (SAMPLE) {
    // counter c = step << 48 | sequence << 32 | n with n < 2^32, so the state
    // seed + (c + 1) * golden advances by THREADS * golden from one n to the next
    const uint64_t base = ((uint64_t)step << 48) | ((uint64_t)(m0 + m) << 32);
    uint64_t state = seed + (base + threadIdx.x + 1) * kGolden64;
    double bv = -INFINITY;
    for (int64_t n = threadIdx.x; n < N; n += THREADS, state += (uint64_t)THREADS * kGolden64) {
      const uint64_t z = splitmix64_mix(state);
      const double u = ((double)(z >> 12) + 0.5) * 0x1p-52;
      const double s = (double)r[n] / temperature - log(-log(u));
      better(bv, bi, s, (int)n);
    }
    block_best<THREADS>(bv, bi);
  } else {
    // four loads in flight per lane before the compares (the loop is latency-bound)
    float bv = -INFINITY;
    int64_t n = threadIdx.x;
    for (; n + 3 * THREADS < N; n += 4 * THREADS) {
      const float v0 = r[n], v1 = r[n + THREADS], v2 = r[n + 2 * THREADS], v3 = r[n + 3 * THREADS];
      better(bv, bi, v0, (int)n);
      better(bv, bi, v1, (int)(n + THREADS));
      better(bv, bi, v2, (int)(n + 2 * THREADS));
      better(bv, bi, v3, (int)(n + 3 * THREADS));
    }
    for (; n < N; n += THREADS) better(bv, bi, r[n], (int)n);
    block_best<THREADS>(bv, bi);
  }
  if (threadIdx.x == 0) {
    const int t = bi == 0x7FFFFFFF ? 0 : bi;
    next[m] = t;
    if (stopped) stopped[m] = (stop >= 0 && t == stop) ? 1 : (fresh ? 0 : stopped[m]);
  }
}

}  // namespace flexq

using namespace flexq;

extern "C" int flexq_layernorm(const uint16_t* x, int64_t M, int64_t h, int64_t x_row_stride,
                               const uint16_t* g, const uint16_t* b, uint16_t* y,
                               hipStream_t stream) {
  if (M < 0 || h <= 0 || h % 8 || h > (int64_t)kLnThreads * 8 * kLnMaxChunks) return FLEXQ_ERR_INVALID;
  if (x_row_stride < h || x_row_stride % 8) return FLEXQ_ERR_INVALID;
  if (M == 0) return FLEXQ_OK;
  if (!x || !g || !b || !y) return FLEXQ_ERR_INVALID;
  if (((uintptr_t)x | (uintptr_t)g | (uintptr_t)b | (uintptr_t)y) & 15) return FLEXQ_ERR_INVALID;
  if (M > 0x7FFFFFFF) return FLEXQ_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(layernorm_kernel, dim3((unsigned)M), dim3(kLnThreads), 0, stream, (const f16*)x,
                     x_row_stride, (int)h, (const f16*)g, (const f16*)b, (f16*)y);
  FLEXQ_LAUNCH_CHECK();
  return FLEXQ_OK;
}

extern "C" int flexq_embed(const int32_t* tokens, int64_t n, int32_t pos_base, int32_t seq,
                           const int32_t* pad, const flexq_w4* embed, const uint16_t* pos,
                           int32_t pos_rows, uint16_t* out, hipStream_t stream) {
  if (n < 0 || !embed || seq <= 0 || pos_base < 0) return FLEXQ_ERR_INVALID;
  if (n == 0) return FLEXQ_OK;
  if (!tokens || !embed->codes || !embed->params || !pos || !out) return FLEXQ_ERR_INVALID;
  const int64_t h = embed->cols;
  if (h <= 0 || h % 64 || embed->rows <= 0) return FLEXQ_ERR_INVALID;
  if ((int64_t)pos_base + (n < seq ? n : seq) - 1 + 2 >= pos_rows) return FLEXQ_ERR_INVALID;
  if (((uintptr_t)embed->codes & 7) || ((uintptr_t)embed->params & 3) || ((uintptr_t)pos & 15) ||
      ((uintptr_t)out & 15) || ((uintptr_t)pad & 3))
    return FLEXQ_ERR_INVALID;
  if (n > 0x7FFFFFFF || embed->rows > 0x7FFFFFFF) return FLEXQ_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(embed_kernel, dim3((unsigned)n), dim3(256), 0, stream, tokens, pos_base, seq,
                     pad, (int)h, (const uint2*)embed->codes, (const uint32_t*)embed->params,
                     (const f16*)pos, pos_rows, (int)embed->rows, (f16*)out);
  FLEXQ_LAUNCH_CHECK();
  return FLEXQ_OK;
}

namespace flexq {

int launch_pick(const float* logits, int64_t M, int64_t N, const flexq_gen_config* gen,
                int32_t step, int32_t m0, int32_t* stopped, bool fresh, int32_t* next,
                hipStream_t stream) {
  if (M < 0 || N <= 0 || N > 0x7FFFFFFF) return FLEXQ_ERR_INVALID;
  if (M == 0) return FLEXQ_OK;
  if (!logits || !next) return FLEXQ_ERR_INVALID;
  if (M > 0x7FFFFFFF) return FLEXQ_ERR_UNSUPPORTED;
  const bool sample = gen && gen->do_sample;
  const int32_t stop = gen ? gen->stop : -1;
  if (gen && stop >= N) return FLEXQ_ERR_INVALID;
  if (stop < 0) stopped = nullptr;
  if (sample) {
    if (!(gen->temperature > 0.0f) || !(gen->temperature <= __FLT_MAX__)) return FLEXQ_ERR_INVALID;
    if (step < 0 || step > 0xFFFF || m0 < 0 || (int64_t)m0 + M > 0x10000) return FLEXQ_ERR_INVALID;
    hipLaunchKernelGGL((pick_kernel<true, 1024>), dim3((unsigned)M), dim3(1024), 0, stream, logits,
                       N, gen->seed, (double)gen->temperature, (uint32_t)step, (uint32_t)m0, stop,
                       stopped, (int)fresh, next);
  } else {
    hipLaunchKernelGGL((pick_kernel<false, 1024>), dim3((unsigned)M), dim3(1024), 0, stream, logits,
                       N, (uint64_t)0, 1.0, 0u, 0u, stop, stopped, (int)fresh, next);
  }
  FLEXQ_LAUNCH_CHECK();
  return FLEXQ_OK;
}

}  // namespace flexq

extern "C" int flexq_argmax(const float* logits, int64_t M, int64_t N, int32_t* next,
                            hipStream_t stream) {
  return launch_pick(logits, M, N, nullptr, 0, 0, nullptr, false, next, stream);
}

extern "C" int flexq_pick(const float* logits, int64_t M, int64_t N, const flexq_gen_config* gen,
                          int32_t step, int32_t m0, int32_t* stopped, int32_t* next,
                          hipStream_t stream) {
  return launch_pick(logits, M, N, gen, step, m0, stopped, false, next, stream);
}
