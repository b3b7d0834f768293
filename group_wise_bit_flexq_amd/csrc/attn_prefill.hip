// Prefill attention (the pages' `mha`, source notes section "Pytorch Backend") with
// the 4-bit KV store fused at the end (walkthrough section 6.3, cache config:
// group 64 along head_dim).
//
// One work-group per (64-query block, head, sequence); 4 waves of 16 queries.
// Key/value blocks of 64 positions are staged in LDS (K row-major, V transposed),
// scores come from v_mfma_f32_16x16x32_f16 as S^T = K . Q^T, an online softmax in
// fp32 (exp2 with the 1/sqrt(hd) * log2(e) factor folded into the scores) keeps a
// running max/sum per query, and O^T += V^T . P^T reuses the score registers
// directly as the B operand: lane (q + 16 g) holds keys 4g..4g+3 of two 16-key
// tiles, so both operands number the 32 keys of a step the same way.
// After the softmax loop the group quantizes K and V of its own 64 positions into
// the cache (8 lanes per 64-element group), reading them back from the qkv rows.
#include "quant_dev.h"

namespace flexq {

struct KVView {
  uint8_t* kc;
  uint8_t* vc;
  uint32_t* kp;
  uint32_t* vp;
  int nh, max_len;
};

template <int HD>
__global__ __launch_bounds__(256) void attn_prefill_kernel(const f16* __restrict__ qkv, int S,
                                                           int nh, int b0, KVView kv,
                                                           f16* __restrict__ out,
                                                           float scale_log2) {
  constexpr int KB = 64;           // keys per block
  constexpr int HC = HD / 8;       // 16-B chunks per K row
  constexpr int VT_LD = KB + 8;    // transposed V row length (halves)
  __shared__ __attribute__((aligned(16))) f16 sK[KB * HD];
  __shared__ __attribute__((aligned(16))) f16 sVt[HD * VT_LD];

  const int nqb = (S + 63) / 64;
  const int qb = nqb - 1 - blockIdx.x;  // long (late) query blocks first
  const int head = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = nh * HD;
  const int64_t ld = 3 * (int64_t)h;
  const f16* base = qkv + (int64_t)b * S * ld;
  const int q0 = qb * 64;
  const int g = lane >> 4;           // lane group 0..3
  const int ql = lane & 15;          // query within the wave's 16
  const int qabs = q0 + wave * 16 + ql;
  const int qrow = min(qabs, S - 1);

  // Q^T operand: lane (q + 16g) holds Q[q][32 ks + 8 g .. +7]
  f16x8 qf[HD / 32];
#pragma unroll
  for (int ks = 0; ks < HD / 32; ++ks)
    qf[ks] = *(const f16x8*)(base + (int64_t)qrow * ld + head * HD + ks * 32 + g * 8);

  f32x4 o[HD / 16];
#pragma unroll
  for (int i = 0; i < HD / 16; ++i) o[i] = (f32x4){0, 0, 0, 0};
  float m_run = -INFINITY, l_run = 0.0f;

  for (int kb = 0; kb <= qb; ++kb) {
    const int k0 = kb * KB;
    __syncthreads();
    // stage K rows (swizzled 16-B chunks) and V transposed
    for (int idx = tid; idx < KB * HC; idx += 256) {
      const int key = idx / HC, ch = idx % HC;
      const int t = k0 + key;
      uint4 kv4 = make_uint4(0, 0, 0, 0), vv4 = make_uint4(0, 0, 0, 0);
      if (t < S) {
        const f16* row = base + (int64_t)t * ld + head * HD + ch * 8;
        kv4 = *(const uint4*)(row + h);
        vv4 = *(const uint4*)(row + 2 * h);
      }
      *(uint4*)(sK + key * HD + ((ch ^ (key & 7)) << 3)) = kv4;
      const f16x8 vh = __builtin_bit_cast(f16x8, vv4);
#pragma unroll
      for (int e = 0; e < 8; ++e) sVt[(ch * 8 + e) * VT_LD + key] = vh[e];
    }
    __syncthreads();

    // S^T tiles: 4 tiles of 16 keys; lane (q + 16g) reg r = key 16 t + 4 g + r
    f32x4 s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[t] = (f32x4){0, 0, 0, 0};
      const int krow = t * 16 + ql;
#pragma unroll
      for (int ks = 0; ks < HD / 32; ++ks) {
        const int ch = ks * 4 + g;
        const f16x8 kf = *(const f16x8*)(sK + krow * HD + ((ch ^ (krow & 7)) << 3));
        s[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[ks], s[t], 0, 0, 0);
      }
    }
    // scale, mask (causal and past the end), block max
    const bool diag = (kb == qb) || (k0 + KB > S);
    float mb = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = s[t][r] * scale_log2;
        if (diag) {
          const int key = k0 + t * 16 + g * 4 + r;
          if (key > qabs || key >= S) v = -INFINITY;
        }
        s[t][r] = v;
        mb = fmaxf(mb, v);
      }
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    const float m_new = fmaxf(m_run, mb);
    const float alpha = exp2f(m_run - m_new);  // m_run = -inf on the first block -> 0
    float ls = 0.0f;
    f16x8 pf[2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(s[t][r] - m_new);
        ls += p;
        pf[t >> 1][(t & 1) * 4 + r] = (f16)p;
      }
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < HD / 16; ++i) o[i] *= alpha;

    // O^T[d][q] += sum over 32-key steps of V^T[d][key] P^T[key][q]
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
      for (int dt = 0; dt < HD / 16; ++dt) {
        const f16* vrow = sVt + (dt * 16 + ql) * VT_LD + kc * 32 + g * 4;
        const f16x4 lo = *(const f16x4*)(vrow);
        const f16x4 hi = *(const f16x4*)(vrow + 16);
        const f16x8 vf = (f16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[kc], o[dt], 0, 0, 0);
      }
    }
  }

  // O^T lane (q + 16 g) reg r = dim 16 dt + 4 g + r of query q
  if (qabs < S) {
    const float inv = 1.0f / l_run;
    f16* orow = out + ((int64_t)b * S + qabs) * h + head * HD;
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt) {
      const f16x4 v = (f16x4){(f16)(o[dt][0] * inv), (f16)(o[dt][1] * inv), (f16)(o[dt][2] * inv),
                              (f16)(o[dt][3] * inv)};
      *(f16x4*)(orow + dt * 16 + g * 4) = v;
    }
  }

  // 4-bit store of K and V for positions [q0, q0 + 64): 8 lanes per group
  constexpr int GPT = HD / 64;                     // groups per token vector
  constexpr int NGROUPS = 64 * GPT * 2;            // K and V
  const int sub = tid & 7;
  for (int gi = tid >> 3; gi < NGROUPS; gi += 32) {
    const int isv = gi / (64 * GPT);
    const int rem = gi % (64 * GPT);
    const int tok = q0 + rem / GPT;
    const int grp = rem % GPT;
    const int tl = min(tok, S - 1);
    const f16* src = base + (int64_t)tl * ld + (1 + isv) * h + head * HD + grp * 64 + sub * 8;
    const f16x8 xv = *(const f16x8*)src;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)xv[e];
    uint32_t packed[1];
    const uint32_t prm = GroupQ<8>::run(x, packed);
    if (tok < S) {
      const int64_t slot = ((int64_t)(b0 + b) * kv.nh + head) * kv.max_len + tok;
      uint8_t* cbase = isv ? kv.vc : kv.kc;
      uint32_t* pbase = isv ? kv.vp : kv.kp;
      *(uint32_t*)(cbase + slot * (HD / 2) + grp * 32 + sub * 4) = packed[0];
      if (sub == 0) pbase[slot * GPT + grp] = prm;
    }
  }
}

}  // namespace flexq

using namespace flexq;

extern "C" int flexq_attn_prefill(const uint16_t* qkv, int32_t B, int32_t S, int32_t b0,
                                  const flexq_kv4_layer* kv, uint16_t* out, hipStream_t stream) {
  if (!kv || !qkv || !out) return FLEXQ_ERR_INVALID;
  if (B < 0 || S < 0 || b0 < 0) return FLEXQ_ERR_INVALID;
  if (B == 0 || S == 0) return FLEXQ_OK;
  if (kv->head_dim != 64 && kv->head_dim != 128) return FLEXQ_ERR_UNSUPPORTED;
  if (kv->heads <= 0 || b0 + B > kv->batch || S > kv->max_len) return FLEXQ_ERR_INVALID;
  if (!kv->k_codes || !kv->v_codes || !kv->k_params || !kv->v_params) return FLEXQ_ERR_INVALID;
  if (((uintptr_t)qkv & 15) || ((uintptr_t)out & 15) || ((uintptr_t)kv->k_codes & 15) ||
      ((uintptr_t)kv->v_codes & 15) || ((uintptr_t)kv->k_params & 3) || ((uintptr_t)kv->v_params & 3))
    return FLEXQ_ERR_INVALID;
  if (kv->heads > 65535 || B > 65535) return FLEXQ_ERR_UNSUPPORTED;
  KVView v{kv->k_codes, kv->v_codes, (uint32_t*)kv->k_params, (uint32_t*)kv->v_params, kv->heads,
           kv->max_len};
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)kv->head_dim);
  dim3 grid((S + 63) / 64, kv->heads, B);
  if (kv->head_dim == 64)
    hipLaunchKernelGGL(attn_prefill_kernel<64>, grid, dim3(256), 0, stream, (const f16*)qkv, S,
                       kv->heads, b0, v, (f16*)out, scale_log2);
  else
    hipLaunchKernelGGL(attn_prefill_kernel<128>, grid, dim3(256), 0, stream, (const f16*)qkv, S,
                       kv->heads, b0, v, (f16*)out, scale_log2);
  FLEXQ_LAUNCH_CHECK();
  return FLEXQ_OK;
}
