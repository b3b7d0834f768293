// Decode attention over the 4-bit KV cache (the pages' `mha_gen`, source notes
// section "Pytorch Backend"; compressed cache per walkthrough section 6.3).
//
// Work-group = (context split, head, sequence), 256 threads.  A token's K (or V)
// vector is head_dim/2 bytes of codes; LPT = head_dim/32 lanes share a token, each
// lane owning 32 fixed dimensions (half a quantization group), so a wave covers
// 64/LPT tokens per step and each lane keeps its slice of q in registers.
//
//  1. the split that ends at `pos` first quantizes this step's k and v (8 lanes per
//     64-element group) and appends them at position pos;
//  2. K pass: score_t = sum_g [ s_g * sum_d q_d c_td + m_g * sum_d q_d ]  (the
//     dequantized key c*s+m never materialises).  Codes enter v_dot2_f32_f16 as fp16
//     subnormals c * 2^-24, so every product is exact and the 2^24 is folded into s;
//  3. softmax over the split in fp32 (two passes over scores kept in LDS);
//  4. V pass: o_d = sum_t p_t s_t c_td + sum_t p_t m_t, fp32 FMAs;
//  5. with several splits, each writes (max, sum, o[]) and a merge kernel rescales
//     and adds them in split order.
// Left padding: positions below the sequence's pad count are never read; a split that
// lies wholly below it writes an empty partial (max -inf, sum 0), which the merge
// weights by 0 (the split holding pos is never empty).
#include <algorithm>

#include "quant_dev.h"

namespace flexq {

struct KVViewD {
  uint8_t* kc;
  uint8_t* vc;
  uint32_t* kp;
  uint32_t* vp;
  int nh, max_len;
};

constexpr int kDecMaxChunk = 4096;  // tokens of one split (scores live in LDS)

// byte N of a word as float (one v_cvt_f32_ubyteN)
template <int N>
__device__ __forceinline__ float byte_f(uint32_t w) { return (float)((w >> (8 * N)) & 0xFFu); }

template <int HD, int UNR>
__global__ __launch_bounds__(256) void attn_decode_kernel(const f16* __restrict__ qkv, int b0,
                                                          int pos, KVViewD kv,
                                                          const int32_t* __restrict__ pad,
                                                          int chunk, f16* __restrict__ out,
                                                          float* __restrict__ part,
                                                          float scale_log2) {
  constexpr int LPT = HD / 32;     // lanes per token
  constexpr int TPW = 64 / LPT;    // tokens per wave step
  constexpr int TPB = 4 * TPW;     // tokens per block step
  constexpr int GPT = HD / 64;     // quantization groups per token vector
  __shared__ float sc[kDecMaxChunk];
  __shared__ float red[4][HD + LPT];
  __shared__ float wred[8];

  const int split = blockIdx.x, head = blockIdx.y, bi = blockIdx.z;
  const int nsplit = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nh = kv.nh;
  const int h = nh * HD;
  const int T = pos + 1;
  const int t_end = min(T, split * chunk + chunk);
  const int npad = pad ? min(max(pad[b0 + bi], 0), pos) : 0;
  const int t_begin = max(split * chunk, npad);
  const f16* row = qkv + (int64_t)bi * 3 * h;
  const int64_t slot0 = ((int64_t)(b0 + bi) * nh + head) * kv.max_len;

  // ---- 1. quantize-append of this step's k, v at position pos
  if (t_end == T) {
    if (wave == 0) {
      const int gi = min(lane >> 3, 2 * GPT - 1);
      const int sub = lane & 7;
      const int isv = gi / GPT, grp = gi % GPT;
      const f16x8 xv = *(const f16x8*)(row + (1 + isv) * h + head * HD + grp * 64 + sub * 8);
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (float)xv[e];
      uint32_t packed[1];
      const uint32_t prm = GroupQ<8>::run(x, packed);
      if ((lane >> 3) < 2 * GPT) {
        uint8_t* cb = isv ? kv.vc : kv.kc;
        uint32_t* pb = isv ? kv.vp : kv.kp;
        *(uint32_t*)(cb + (slot0 + pos) * (HD / 2) + grp * 32 + sub * 4) = packed[0];
        if (sub == 0) pb[(slot0 + pos) * GPT + grp] = prm;
      }
    }
  }
  // only this work-group reads position pos in this launch: the barrier's
  // work-group-scope release/acquire orders the append before the reads below
  __syncthreads();

  // ---- this lane's slice of q: dims 32 j .. 32 j + 31 (group j / 2)
  const int j = lane % LPT;
  const int grp = j >> 1;
  f16x2 q2[16];
  float qsum = 0.0f;
  {
    const uint4* qp = (const uint4*)(row + head * HD + 32 * j);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 u = qp[c];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        q2[c * 4 + k] = h2_from_u32(w[k]);
        qsum += (float)q2[c * 4 + k].x + (float)q2[c * 4 + k].y;
      }
    }
  }

  // ---- 2. K pass, UNR block steps per iteration: every load of the iteration is
  // issued before the first use (token index clamped to the split's last token, the
  // results of clamped lanes discarded), so UNR x 20 B per lane are in flight
  for (int tb = t_begin; tb < t_end; tb += UNR * TPB) {
    uint4 cw[UNR];
    uint32_t prm[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int t = min(tb + u * TPB + wave * TPW + lane / LPT, t_end - 1);
      cw[u] = *(const uint4*)(kv.kc + (slot0 + t) * (HD / 2) + 16 * j);
      prm[u] = kv.kp[(slot0 + t) * GPT + grp];
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int t = tb + u * TPB + wave * TPW + lane / LPT;
      const uint32_t w[4] = {cw[u].x, cw[u].y, cw[u].z, cw[u].w};
      float dot = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = w[k] & 0x0F0F0F0Fu, hi = (w[k] >> 4) & 0x0F0F0F0Fu;
        // code pairs as fp16 subnormals c * 2^-24, element order (2i, 2i+1)
        dot = __builtin_amdgcn_fdot2(h2_from_u32(__builtin_amdgcn_perm(hi, lo, 0x0c040c00u)), q2[4 * k + 0], dot, false);
        dot = __builtin_amdgcn_fdot2(h2_from_u32(__builtin_amdgcn_perm(hi, lo, 0x0c050c01u)), q2[4 * k + 1], dot, false);
        dot = __builtin_amdgcn_fdot2(h2_from_u32(__builtin_amdgcn_perm(hi, lo, 0x0c060c02u)), q2[4 * k + 2], dot, false);
        dot = __builtin_amdgcn_fdot2(h2_from_u32(__builtin_amdgcn_perm(hi, lo, 0x0c070c03u)), q2[4 * k + 3], dot, false);
      }
      const float m = (float)h_from_bits(prm[u] & 0xFFFFu);
      const float s = (float)h_from_bits(prm[u] >> 16);
      float partial = (s * 16777216.0f) * dot + m * qsum;
#pragma unroll
      for (int o = 1; o < LPT; o <<= 1) partial += __shfl_xor(partial, o, 64);
      if (j == 0 && t < t_end) sc[t - t_begin] = partial * scale_log2;
    }
  }
  __syncthreads();

  // ---- 3. softmax statistics of this split
  const int n = t_end - t_begin;   // <= 0 for a split wholly in the padding
  float mx = -INFINITY;
  for (int i = tid; i < n; i += 256) mx = fmaxf(mx, sc[i]);
  mx = wave_max(mx);
  if (lane == 0) wred[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
  float ls = 0.0f;
  for (int i = tid; i < n; i += 256) {
    const float p = exp2f(sc[i] - mx);
    sc[i] = p;
    ls += p;
  }
  ls = wave_sum(ls);
  __syncthreads();
  if (lane == 0) wred[4 + wave] = ls;
  __syncthreads();
  const float lsum = (wred[4] + wred[5]) + (wred[6] + wred[7]);

  // ---- 4. V pass
  float acc[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) acc[e] = 0.0f;
  float pm = 0.0f;
  for (int tb = t_begin; tb < t_end; tb += UNR * TPB) {
    uint4 cw[UNR];
    uint32_t prm[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int t = min(tb + u * TPB + wave * TPW + lane / LPT, t_end - 1);
      cw[u] = *(const uint4*)(kv.vc + (slot0 + t) * (HD / 2) + 16 * j);
      prm[u] = kv.vp[(slot0 + t) * GPT + grp];
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int t = tb + u * TPB + wave * TPW + lane / LPT;
      // clamped lanes repeat the last token: their weight is zero
      const float p = t < t_end ? sc[t - t_begin] : 0.0f;
      const float m = (float)h_from_bits(prm[u] & 0xFFFFu);
      const float s = (float)h_from_bits(prm[u] >> 16);
      const float ps = p * s;
      pm += p * m;
      const uint32_t w[4] = {cw[u].x, cw[u].y, cw[u].z, cw[u].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = w[k] & 0x0F0F0F0Fu, hi = (w[k] >> 4) & 0x0F0F0F0Fu;
        acc[8 * k + 0] += ps * byte_f<0>(lo);
        acc[8 * k + 1] += ps * byte_f<0>(hi);
        acc[8 * k + 2] += ps * byte_f<1>(lo);
        acc[8 * k + 3] += ps * byte_f<1>(hi);
        acc[8 * k + 4] += ps * byte_f<2>(lo);
        acc[8 * k + 5] += ps * byte_f<2>(hi);
        acc[8 * k + 6] += ps * byte_f<3>(lo);
        acc[8 * k + 7] += ps * byte_f<3>(hi);
      }
    }
  }
  // lanes of one wave that own the same dims: xor over the token bits of the lane id
#pragma unroll
  for (int o = LPT; o < 64; o <<= 1) {
#pragma unroll
    for (int e = 0; e < 32; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
    pm += __shfl_xor(pm, o, 64);
  }
  if (lane < LPT) {
#pragma unroll
    for (int e = 0; e < 32; ++e) red[wave][32 * lane + e] = acc[e];
    red[wave][HD + lane] = pm;
  }
  __syncthreads();

  // ---- 5. output (one thread per dim)
  if (tid < HD) {
    const int d = tid, pj = d / 32;
    const float od = ((red[0][d] + red[1][d]) + (red[2][d] + red[3][d])) +
                     ((red[0][HD + pj] + red[1][HD + pj]) + (red[2][HD + pj] + red[3][HD + pj]));
    if (nsplit == 1) {
      out[(int64_t)bi * h + head * HD + d] = (f16)(od / lsum);
    } else {
      float* pp = part + (((int64_t)bi * nh + head) * nsplit + split) * (HD + 2);
      pp[2 + d] = od;
      if (d == 0) {
        pp[0] = mx;
        pp[1] = lsum;
      }
    }
  }
}

// Merge of split partials (max m_z, sum l_z, unnormalised o_z): fixed split order.
template <int HD>
__global__ __launch_bounds__(HD) void attn_decode_merge_kernel(const float* __restrict__ part,
                                                               int nsplit, int nh,
                                                               f16* __restrict__ out) {
  const int head = blockIdx.x, bi = blockIdx.y, d = threadIdx.x;
  const float* pp = part + ((int64_t)bi * nh + head) * nsplit * (HD + 2);
  float M = -INFINITY;
  for (int z = 0; z < nsplit; ++z) M = fmaxf(M, pp[z * (HD + 2)]);
  float L = 0.0f, o = 0.0f;
  for (int z = 0; z < nsplit; ++z) {
    const float w = exp2f(pp[z * (HD + 2)] - M);
    L += pp[z * (HD + 2) + 1] * w;
    o += pp[z * (HD + 2) + 2 + d] * w;
  }
  out[(int64_t)bi * nh * HD + head * HD + d] = (f16)(o / L);
}

struct DecPlan {
  int splits, chunk, unr;
};

// Unroll of the token loops: the largest of 4, 3, 2 that wastes at most 1/8 of the
// block steps of a split on clamped lanes, else 1.
static int dec_unroll(int steps) {
  for (int u = 4; u >= 2; --u)
    if (((steps + u - 1) / u * u - steps) * 8 <= steps) return u;
  return 1;
}

static DecPlan dec_plan(int B, int heads, int head_dim, int pos) {
  const int T = pos + 1;
  const int step = head_dim == 128 ? 64 : 128;  // tokens per block step
  const int pairs = B * heads;
  int splits = (1024 + pairs - 1) / pairs;
  splits = std::max(1, std::min(splits, (T + step - 1) / step));
  splits = std::max(splits, (T + kDecMaxChunk - 1) / kDecMaxChunk);
  int chunk = (T + splits - 1) / splits;
  chunk = (chunk + step - 1) / step * step;
  if (chunk > kDecMaxChunk) chunk = kDecMaxChunk;
  const int nsplit = (T + chunk - 1) / chunk;
  // the longest split decides; shorter (last) splits only clamp more lanes
  DecPlan p{nsplit, chunk, dec_unroll((std::min(chunk, T) + step - 1) / step)};
  return p;
}

template <int HD, int UNR>
static void launch_dec(const DecPlan& p, dim3 grid, const f16* qkv, int b0, int pos,
                       const KVViewD& v, const int32_t* pad, f16* out, float* ws,
                       float scale_log2, hipStream_t stream) {
  hipLaunchKernelGGL((attn_decode_kernel<HD, UNR>), grid, dim3(256), 0, stream, qkv, b0, pos, v,
                     pad, p.chunk, out, ws, scale_log2);
}

template <int HD>
static void launch_dec(const DecPlan& p, dim3 grid, const f16* qkv, int b0, int pos,
                       const KVViewD& v, const int32_t* pad, f16* out, float* ws,
                       float scale_log2, hipStream_t stream) {
  switch (p.unr) {
    case 4: launch_dec<HD, 4>(p, grid, qkv, b0, pos, v, pad, out, ws, scale_log2, stream); break;
    case 3: launch_dec<HD, 3>(p, grid, qkv, b0, pos, v, pad, out, ws, scale_log2, stream); break;
    case 2: launch_dec<HD, 2>(p, grid, qkv, b0, pos, v, pad, out, ws, scale_log2, stream); break;
    default: launch_dec<HD, 1>(p, grid, qkv, b0, pos, v, pad, out, ws, scale_log2, stream); break;
  }
}

}  // namespace flexq

using namespace flexq;

extern "C" size_t flexq_attn_decode_workspace_size(int32_t B, int32_t heads, int32_t head_dim,
                                                   int32_t pos) {
  if (B <= 0 || heads <= 0 || pos < 0 || (head_dim != 64 && head_dim != 128)) return 0;
  const DecPlan p = dec_plan(B, heads, head_dim, pos);
  if (p.splits <= 1) return 0;
  return (size_t)B * heads * p.splits * (head_dim + 2) * sizeof(float);
}

extern "C" int flexq_attn_decode_kv4(const uint16_t* qkv, int32_t B, int32_t b0, int32_t pos,
                                     const flexq_kv4_layer* kv, uint16_t* out, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  if (!kv || !qkv || !out) return FLEXQ_ERR_INVALID;
  if (B < 0 || b0 < 0 || pos < 0) return FLEXQ_ERR_INVALID;
  if (B == 0) return FLEXQ_OK;
  if (kv->head_dim != 64 && kv->head_dim != 128) return FLEXQ_ERR_UNSUPPORTED;
  if (kv->heads <= 0 || b0 + B > kv->batch || pos >= kv->max_len) return FLEXQ_ERR_INVALID;
  if (!kv->k_codes || !kv->v_codes || !kv->k_params || !kv->v_params) return FLEXQ_ERR_INVALID;
  if (((uintptr_t)qkv & 15) || ((uintptr_t)out & 1) || ((uintptr_t)kv->k_codes & 15) ||
      ((uintptr_t)kv->v_codes & 15) || ((uintptr_t)kv->k_params & 3) || ((uintptr_t)kv->v_params & 3) ||
      ((uintptr_t)kv->pad & 3))
    return FLEXQ_ERR_INVALID;
  if (kv->heads > 65535 || B > 65535) return FLEXQ_ERR_UNSUPPORTED;
  const DecPlan p = dec_plan(B, kv->heads, kv->head_dim, pos);
  const size_t need = flexq_attn_decode_workspace_size(B, kv->heads, kv->head_dim, pos);
  if (need > 0 && (!ws || ws_bytes < need || ((uintptr_t)ws & 15))) return FLEXQ_ERR_INVALID;
  KVViewD v{kv->k_codes, kv->v_codes, (uint32_t*)kv->k_params, (uint32_t*)kv->v_params, kv->heads,
            kv->max_len};
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)kv->head_dim);
  dim3 grid(p.splits, kv->heads, B);
  if (kv->head_dim == 64) {
    launch_dec<64>(p, grid, (const f16*)qkv, b0, pos, v, kv->pad, (f16*)out, (float*)ws,
                   scale_log2, stream);
    if (p.splits > 1)
      hipLaunchKernelGGL(attn_decode_merge_kernel<64>, dim3(kv->heads, B), dim3(64), 0, stream,
                         (const float*)ws, p.splits, kv->heads, (f16*)out);
  } else {
    launch_dec<128>(p, grid, (const f16*)qkv, b0, pos, v, kv->pad, (f16*)out, (float*)ws,
                    scale_log2, stream);
    if (p.splits > 1)
      hipLaunchKernelGGL(attn_decode_merge_kernel<128>, dim3(kv->heads, B), dim3(128), 0, stream,
                         (const float*)ws, p.splits, kv->heads, (f16*)out);
  }
  FLEXQ_LAUNCH_CHECK();
  return FLEXQ_OK;
}
