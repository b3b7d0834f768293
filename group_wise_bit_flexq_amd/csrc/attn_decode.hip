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
//     dequantized key c*s+m never materialises).  Codes enter as fp16 subnormals
//     c * 2^-24, so every product is exact and the 2^24 is folded into s; with
//     head_dim 128 the sums run on the matrix cores (q as a 4-row A operand), with 64
//     in v_dot2_f32_f16;
//  3. softmax over the split in fp32: the maximum is kept during the K pass, then one
//     pass over the scores in LDS turns them into weights and sums them;
//  4. V pass: o_d = sum_t p_t s_t c_td + sum_t p_t m_t, fp32 FMAs (v_fma_mix) reading
//     the codes as fp16 subnormals, two per byte permute, as in the K pass;
//  5. with several splits, each writes (max, sum, o[]) and a merge kernel rescales
//     and adds them in split order.
// The K and V rows of one (sequence, head) are read through raw buffer views that end
// at the split's last position, so lanes past the end read zeros and are discarded.
// Left padding: positions below the sequence's pad count are never read; a split that
// lies wholly below it writes an empty partial (max -inf, sum 0), which the merge
// weights by 0 (the split holding pos is never empty).
// Sparse variant (TOPK, one split per sequence and head): after the K pass the n scores
// in LDS are cut to the k = ceil(sparsity * n) largest (a 4-pass radix select over
// order-preserving 32-bit keys, equal keys ranked by position), the others become
// -inf, and the V pass walks a compacted list of the kept positions only.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "host_cache.h"
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

// Float -> uint32 with the same order (negative values reversed below the positives).
__device__ __forceinline__ uint32_t ord_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Keep the kk largest of sc[0, n) (kk < n; lower index first among equal values) and
// set the others to -inf.  All 256 threads of the work-group call it; it ends with a
// barrier.
__device__ void topk_mask(float* sc, int n, int kk) {
  __shared__ uint32_t hist[256];
  __shared__ int pick[3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t prefix = 0, pmask = 0;
  int need = kk;  // rank from the top, among keys that match the prefix, of the threshold
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    if (shift == 24) {
      // the top byte is the sign and most of the exponent: the scores of one query share
      // a handful of values, so each wave adds one count per distinct bin (a leader
      // lane per bin) instead of 64 colliding atomics
      for (int c = 0; c < n; c += 256) {
        const int i = c + tid;
        const bool valid = i < n;
        const uint32_t bin = valid ? ord_key(sc[i]) >> 24 : 0u;
        uint64_t todo = __ballot(valid);
        while (todo) {
          const int leader = __ffsll((long long)todo) - 1;
          const uint32_t lb = __shfl(bin, leader, 64);
          const uint64_t same = __ballot(valid && bin == lb) & todo;
          if (lane == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(same));
          todo &= ~same;
        }
      }
    } else {
      for (int i = tid; i < n; i += 256) {
        const uint32_t key = ord_key(sc[i]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds digits 255 - 4l .. 252 - 4l (largest first); counts above a lane
      // come from an exclusive scan over the lanes
      const int d0 = 255 - 4 * lane;
      const int c0 = (int)hist[d0], c1 = (int)hist[d0 - 1], c2 = (int)hist[d0 - 2],
                c3 = (int)hist[d0 - 3];
      const int tot = c0 + c1 + c2 + c3;
      int incl = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      int above = incl - tot;
      if (above < need && need <= incl) {
        int d = d0, c = c0;
        if (above + c0 < need) {
          above += c0; d = d0 - 1; c = c1;
          if (above + c1 < need) {
            above += c1; d = d0 - 2; c = c2;
            if (above + c2 < need) { above += c2; d = d0 - 3; c = c3; }
          }
        }
        pick[0] = d;
        pick[1] = need - above;
        pick[2] = c;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)pick[0] << shift;
    pmask |= 255u << shift;
    need = pick[1];
    // every key in the chosen bin is kept: the digits so far already decide the cut
    if (need == pick[2]) break;
  }
  // keys whose digits so far exceed the prefix stay; of those equal to it, `need` of
  // pick[2] stay (all of them after an early exit, else the lowest positions)
  const uint32_t thr = prefix;
  const bool all_equal_kept = need == pick[2];
  for (int i = tid; i < n; i += 256)
    if ((ord_key(sc[i]) & pmask) < thr) sc[i] = -INFINITY;
  __syncthreads();
  if (!all_equal_kept && wave == 0) {   // rank equal keys by position
    int run = 0;
    for (int c = 0; c < n; c += 64) {
      const int i = c + lane;
      const bool e = i < n && sc[i] != -INFINITY && (ord_key(sc[i]) & pmask) == thr;
      const uint64_t bal = __ballot(e);
      const int rank = run + __popcll(bal & ((1ull << lane) - 1ull));
      if (e && rank >= need) sc[i] = -INFINITY;
      run += __popcll(bal);
    }
  }
  __syncthreads();
}

// Indices (into sc) of the entries topk_mask kept, in increasing order, into list;
// wave 0 walks the scores in 64-wide chunks (ballot + prefix count).  Ends with a
// barrier.
__device__ void topk_compact(const float* sc, int n, uint16_t* list) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 64) {
    int run = 0;
    for (int c = 0; c < n; c += 64) {
      const int i = c + lane;
      const bool keep = i < n && sc[i] != -INFINITY;
      const uint64_t bal = __ballot(keep);
      if (keep) list[run + __popcll(bal & ((1ull << lane) - 1ull))] = (uint16_t)i;
      run += __popcll(bal);
    }
  }
  __syncthreads();
}

// Sum of x over the N (1, 2 or 4) consecutive lanes of an aligned group (DPP quad
// permutations: lane ^ 1, then lane ^ 2).
template <int N>
__device__ __forceinline__ float quad_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4, "lanes per token");
  if constexpr (N >= 2)
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
  if constexpr (N >= 4)
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
  return x;
}

// Sum of x over the lanes of a 16-lane row whose index agrees with this lane's modulo
// STEP (DPP row rotations; every such lane ends with the same sum).
template <int STEP>
__device__ __forceinline__ float row_sum_stride(float x) {
  if constexpr (STEP < 16) {
    constexpr int kRowRor = 0x120 + STEP;  // DPP row_ror:STEP
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), kRowRor, 0xF, 0xF, true));
    return row_sum_stride<STEP * 2>(x);
  } else {
    return x;
  }
}

template <int HD, int UNR, bool TOPK>
__global__ __launch_bounds__(256) void attn_decode_kernel(const f16* __restrict__ qkv, int b0,
                                                          int pos, KVViewD kv,
                                                          const int32_t* __restrict__ pad,
                                                          int chunk, f16* __restrict__ out,
                                                          float* __restrict__ part,
                                                          float scale_log2, float sparsity) {
  constexpr int LPT = HD / 32;     // lanes per token
  constexpr int TPW = 64 / LPT;    // tokens per wave step
  constexpr int TPB = 4 * TPW;     // tokens per block step
  constexpr int GPT = HD / 64;     // quantization groups per token vector
  // dynamic LDS: the split's scores (chunk floats), then for top-k the kept list
  extern __shared__ __attribute__((aligned(16))) float sc[];
  __shared__ float red[16][HD + LPT];   // per 16-lane row: V sums and offset terms
  __shared__ float wred[8];

  const int split = blockIdx.x, head = blockIdx.y, bi = blockIdx.z;
  const int nsplit = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nh = kv.nh;
  const int h = nh * HD;
  const int T = pos + 1;
  const int t_end = min(T, split * chunk + chunk);
  const int npad = pad ? min(max(pad[b0 + bi], 0), pos) : 0;
  const int t_begin = max(split * chunk, npad);
  const f16* row = qkv + (int64_t)bi * 3 * h;
  const int64_t slot0 = ((int64_t)(b0 + bi) * nh + head) * kv.max_len;
  // raw buffer views of this (sequence, head)'s rows [0, t_end): a load past the end
  // returns zeros, so the token loops address positions without clamping them
  const rsrc_t k_rs = make_rsrc(kv.kc + slot0 * (HD / 2), t_end * (HD / 2));
  const rsrc_t kp_rs = make_rsrc(kv.kp + slot0 * GPT, t_end * GPT * 4);
  const rsrc_t v_rs = make_rsrc(kv.vc + slot0 * (HD / 2), t_end * (HD / 2));
  const rsrc_t vp_rs = make_rsrc(kv.vp + slot0 * GPT, t_end * GPT * 4);

  const int j = lane % LPT;       // this lane's 32 dims: 32 j .. 32 j + 31 (group j / 2)
  const int grp = j >> 1;
  // K-pass lane map.  With head_dim 128 the dot products go to the matrix cores: lane l
  // holds dims 32 (l / 16) .. +31 of token l % 16 of its wave step, which is the B
  // operand of v_mfma_f32_16x16x32_f16 (k-chunk l / 16, column l % 16); head_dim 64
  // keeps v_dot2 with the V pass's map.
  constexpr bool kMfK = HD == 128;
  const int jk = kMfK ? (lane >> 4) : j;
  const int tk = kMfK ? (lane & 15) : lane / LPT;
  // q and the first batch of K go out before the append: none of these loads can read
  // position pos unless the first batch reaches it (then the batch waits for the append)
  uint4 qraw[4];
  {
    const uint4* qp = (const uint4*)(row + head * HD + 32 * jk);
#pragma unroll
    for (int c = 0; c < 4; ++c) qraw[c] = qp[c];
  }
  u32x4 cw[UNR];
  uint32_t prm[UNR];
  u32x2 kprm[UNR];   // matrix-core K pass: the (offset, scale) words of both groups
  auto load_k = [&](int tb) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int t = tb + u * TPB + wave * TPW + tk;   // >= t_end: zeros
      cw[u] = __builtin_amdgcn_raw_buffer_load_b128(k_rs, t * (HD / 2) + 16 * jk, 0, 0);
      if constexpr (kMfK)
        kprm[u] = __builtin_amdgcn_raw_buffer_load_b64(kp_rs, t * GPT * 4, 0, 0);
      else
        prm[u] = __builtin_amdgcn_raw_buffer_load_b32(kp_rs, (t * GPT + grp) * 4, 0, 0);
    }
  };
  const bool k_early = t_begin < t_end && (t_end < T || t_begin + UNR * TPB <= pos);
  if (k_early) load_k(t_begin);

  // ---- 1. quantize-append of this step's k, v at position pos
  if (t_end == T) {
    if (wave == 0) {
      const int gi = min(lane >> 3, 2 * GPT - 1);
      const int sub = lane & 7;
      const int isv = gi / GPT, ag = gi % GPT;   // K or V, group within the head
      const f16x8 x[1] = {*(const f16x8*)(row + (1 + isv) * h + head * HD + ag * 64 + sub * 8)};
      uint32_t packed[1];
      const uint32_t aprm = GroupQ<8>::run(x, packed);
      if ((lane >> 3) < 2 * GPT) {
        uint8_t* cb = isv ? kv.vc : kv.kc;
        uint32_t* pb = isv ? kv.vp : kv.kp;
        *(uint32_t*)(cb + (slot0 + pos) * (HD / 2) + ag * 32 + sub * 4) = packed[0];
        if (sub == 0) pb[(slot0 + pos) * GPT + ag] = aprm;
      }
    }
  }
  // only this work-group reads position pos in this launch: the barrier's
  // work-group-scope release/acquire orders the append before the reads below
  __syncthreads();

  // q pairs in the order the K pass forms code pairs: for the 8 dims of word k,
  // qe[2k] = (q0, q2), qe[2k+1] = (q4, q6), qo[2k] = (q1, q3), qo[2k+1] = (q5, q7)
  f16x2 qe[8], qo[8];
  float qsum = 0.0f;
  {
    const f16x2 ones = {(f16)1.0f, (f16)1.0f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 u = qraw[c];
      const f16x2 a = h2_from_u32(u.x), b = h2_from_u32(u.y), cc = h2_from_u32(u.z),
                  d = h2_from_u32(u.w);
      qe[2 * c] = f16x2{a.x, b.x};
      qe[2 * c + 1] = f16x2{cc.x, d.x};
      qo[2 * c] = f16x2{a.y, b.y};
      qo[2 * c + 1] = f16x2{cc.y, d.y};
      qsum = __builtin_amdgcn_fdot2(a, ones, qsum, false);   // q * 1 is exact
      qsum = __builtin_amdgcn_fdot2(b, ones, qsum, false);
      qsum = __builtin_amdgcn_fdot2(cc, ones, qsum, false);
      qsum = __builtin_amdgcn_fdot2(d, ones, qsum, false);
    }
  }

  // scores in log2 units: the softmax scale folded into the per-token step (with the
  // 2^24 of the subnormal codes) and into the sum of q for the offset term
  const float ks = 16777216.0f * scale_log2;
  const float qsum_s = qsum * scale_log2;
  // matrix-core K pass.  A word's codes enter as fp16 subnormals, as in the v_dot2
  // pass: even dims c 2^-24 from the low nibbles, odd dims 16 c 2^-24 from the high
  // nibbles left in place, in the order (d0, d2, d4, d6, d1, d3, d5, d7).  A operand
  // rows: 0 = q of group 0's even dims (k-chunks 0, 1; zeros in the odd slots), 1 = the
  // same for group 1 (k-chunks 2, 3), 2 and 3 = the odd dims of groups 0 and 1; every
  // other row is zero.  C rows 0..3 of a token then hold exact-product sums whose odd
  // rows carry a factor 16.  qg0, qg1: the groups' sums of q.
  f16x8 aq[4];
  float qg0 = 0.0f, qg1 = 0.0f;
  if constexpr (kMfK) {
    const int arow = lane & 15, grp_k = jk >> 1;
    const bool even_row = arow == grp_k, odd_row = arow == 2 + grp_k;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f16 z = (f16)0.0f;
      const f16x8 ve = {qe[2 * k].x, qe[2 * k].y, qe[2 * k + 1].x, qe[2 * k + 1].y, z, z, z, z};
      const f16x8 vo = {z, z, z, z, qo[2 * k].x, qo[2 * k].y, qo[2 * k + 1].x, qo[2 * k + 1].y};
      aq[k] = even_row ? ve : (odd_row ? vo : (f16x8){});
    }
    // lanes of 16-lane row r hold the sum of dims 32 r .. 32 r + 31
    const float pair = qsum + __shfl_xor(qsum, 16, 64);   // rows 0, 1: group 0; 2, 3: group 1
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair),
                                                    false, false);
    qg0 = __uint_as_float(r[0]) * scale_log2;
    qg1 = __uint_as_float(r[1]) * scale_log2;
  }

  // ---- 2. K pass, UNR block steps per iteration: every load of the iteration is
  // issued before the first use (positions past the split's end read zeros and their
  // results are discarded), so UNR x 20 B per lane are in flight.  Each lane also
  // keeps the running maximum of its scores for the softmax.
  float mx_run = -INFINITY;
  for (int tb = t_begin; tb < t_end; tb += UNR * TPB) {
    if (!k_early || tb != t_begin) load_k(tb);
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int t = tb + u * TPB + wave * TPW + tk;
      const uint32_t w[4] = {cw[u].x, cw[u].y, cw[u].z, cw[u].w};
      if constexpr (kMfK) {
        f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t lo = w[k] & 0x0F0F0F0Fu, hi = w[k] & 0xF0F0F0F0u;
          const uint32_t b0 = __builtin_amdgcn_perm(lo, lo, 0x0c010c00u);
          const uint32_t b1 = __builtin_amdgcn_perm(lo, lo, 0x0c030c02u);
          const uint32_t b2 = __builtin_amdgcn_perm(hi, hi, 0x0c010c00u);
          const uint32_t b3 = __builtin_amdgcn_perm(hi, hi, 0x0c030c02u);
          const f16x8 b = __builtin_bit_cast(f16x8, (u32x4){b0, b1, b2, b3});
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[k], b, c, 0, 0, 0);
        }
        // lanes 0..15 (token tk): group g's sum of q . c is 2^24 (c[g] + c[2 + g] / 16)
        const float m0 = (float)h_from_bits(kprm[u].x & 0xFFFFu);
        const float s0 = (float)h_from_bits(kprm[u].x >> 16);
        const float m1 = (float)h_from_bits(kprm[u].y & 0xFFFFu);
        const float s1 = (float)h_from_bits(kprm[u].y >> 16);
        const float d0 = __builtin_fmaf(c[2], 0.0625f, c[0]);
        const float d1 = __builtin_fmaf(c[3], 0.0625f, c[1]);
        const float partial = (s0 * ks) * d0 + (s1 * ks) * d1 + (m0 * qg0 + m1 * qg1);
        if (lane < 16 && t < t_end) {
          mx_run = fmaxf(mx_run, partial);
          sc[t - t_begin] = partial;
        }
        continue;
      }
      // code pairs as fp16 subnormals: even dims c * 2^-24 from the low nibbles, odd
      // dims 16 c * 2^-24 from the high nibbles left in place (exact products; the
      // odd-dim sum is scaled by 1/16 once per token)
      float dlo = 0.0f, dhi = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = w[k] & 0x0F0F0F0Fu, hi = w[k] & 0xF0F0F0F0u;
        dlo = __builtin_amdgcn_fdot2(h2_from_u32(__builtin_amdgcn_perm(lo, lo, 0x0c010c00u)), qe[2 * k], dlo, false);
        dlo = __builtin_amdgcn_fdot2(h2_from_u32(__builtin_amdgcn_perm(lo, lo, 0x0c030c02u)), qe[2 * k + 1], dlo, false);
        dhi = __builtin_amdgcn_fdot2(h2_from_u32(__builtin_amdgcn_perm(hi, hi, 0x0c010c00u)), qo[2 * k], dhi, false);
        dhi = __builtin_amdgcn_fdot2(h2_from_u32(__builtin_amdgcn_perm(hi, hi, 0x0c030c02u)), qo[2 * k + 1], dhi, false);
      }
      const float dot = __builtin_fmaf(dhi, 0.0625f, dlo);
      const float m = (float)h_from_bits(prm[u] & 0xFFFFu);
      const float s = (float)h_from_bits(prm[u] >> 16);
      float partial = (s * ks) * dot + m * qsum_s;
      partial = quad_sum<LPT>(partial);
      if (t < t_end) mx_run = fmaxf(mx_run, partial);
      if (j == 0 && t < t_end) sc[t - t_begin] = partial;
    }
  }
  mx_run = wave_max(mx_run);
  if (lane == 0) wred[wave] = mx_run;
  __syncthreads();

  const int n = t_end - t_begin;   // <= 0 for a split wholly in the padding
  // V pass positions: t_begin + j for j < cnt, or t_begin + list[j] for a top-k cut
  int cnt = n;
  bool use_list = false;
  uint16_t* const list = (uint16_t*)(sc + chunk);
  if constexpr (TOPK) {            // one split: n >= 1 candidates
    const int kk = max((int)ceilf(fminf(sparsity, 1.0f) * (float)n), 1);
    if (kk < n) {
      topk_mask(sc, n, kk);
      topk_compact(sc, n, list);
      cnt = kk;
      use_list = true;
    }
  }

  // the dense kernel issues its first batch of V before the softmax statistics
  const bool v_early = !TOPK && cnt > 0;
  int rel[UNR];
  auto load_v = [&](int jb, auto with_list) {
    constexpr bool LIST = decltype(with_list)::value;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int jr = jb + u * TPB + wave * TPW + lane / LPT;
      const int jj = min(jr, cnt - 1);
      rel[u] = LIST ? (int)list[jj] : jj;   // where this lane's p sits in LDS
      // the position read: past the end (dense walk) the loads return zeros
      const int t = t_begin + (LIST ? rel[u] : jr);
      cw[u] = __builtin_amdgcn_raw_buffer_load_b128(v_rs, t * (HD / 2) + 16 * j, 0, 0);
      prm[u] = __builtin_amdgcn_raw_buffer_load_b32(vp_rs, (t * GPT + grp) * 4, 0, 0);
    }
  };
  if (v_early) load_v(0, std::false_type{});

  // ---- 3. softmax statistics of this split (the maximum comes from the K pass; a
  // top-k cut keeps the largest score, so the maximum is the same)
  const float mx = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
  float ls = 0.0f;
  for (int i = tid; i < n; i += 256) {
    // v_exp_f32 as is: arguments are <= 0, and only weights below 2^-126 (nothing
    // next to the maximum's 1) lose their subnormal tail
    const float p = __builtin_amdgcn_exp2f(sc[i] - mx);
    sc[i] = p;
    ls += p;
  }
  ls = wave_sum(ls);
  __syncthreads();
  if (lane == 0) wred[4 + wave] = ls;
  __syncthreads();
  const float lsum = (wred[4] + wred[5]) + (wred[6] + wred[7]);

  // ---- 4. V pass (instantiated with and without the kept list)
  float acc[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) acc[e] = 0.0f;
  float pm = 0.0f;
  auto v_pass = [&](auto with_list) {
    for (int jb = 0; jb < cnt; jb += UNR * TPB) {
      if (!v_early || jb != 0) load_v(jb, with_list);
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        // lanes past the end of the walk: weight zero (their loads read zeros, or
        // repeat the last kept position)
        const bool live = jb + u * TPB + wave * TPW + lane / LPT < cnt;
        const float p = live ? sc[rel[u]] : 0.0f;
        const float m = (float)h_from_bits(prm[u] & 0xFFFFu);
        const float s = (float)h_from_bits(prm[u] >> 16);
        // the codes enter as fp16 subnormals c 2^-24 (even dims, low nibbles) and
        // 16 c 2^-24 (odd dims, high nibbles in place), two per byte permute; 2^24 is
        // folded into the weight, so even-dim products are exactly p s c and odd-dim
        // ones exactly 16 p s c (the odd accumulators are scaled by 1/16 after the pass)
        const float ps = p * s * 16777216.0f;
        pm += p * m;
        const uint32_t w[4] = {cw[u].x, cw[u].y, cw[u].z, cw[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t lo = w[k] & 0x0F0F0F0Fu, hi = w[k] & 0xF0F0F0F0u;
          const f16x2 e02 = h2_from_u32(__builtin_amdgcn_perm(lo, lo, 0x0c010c00u));
          const f16x2 e46 = h2_from_u32(__builtin_amdgcn_perm(lo, lo, 0x0c030c02u));
          const f16x2 e13 = h2_from_u32(__builtin_amdgcn_perm(hi, hi, 0x0c010c00u));
          const f16x2 e57 = h2_from_u32(__builtin_amdgcn_perm(hi, hi, 0x0c030c02u));
          acc[8 * k + 0] = __builtin_fmaf(ps, (float)e02.x, acc[8 * k + 0]);
          acc[8 * k + 1] = __builtin_fmaf(ps, (float)e13.x, acc[8 * k + 1]);
          acc[8 * k + 2] = __builtin_fmaf(ps, (float)e02.y, acc[8 * k + 2]);
          acc[8 * k + 3] = __builtin_fmaf(ps, (float)e13.y, acc[8 * k + 3]);
          acc[8 * k + 4] = __builtin_fmaf(ps, (float)e46.x, acc[8 * k + 4]);
          acc[8 * k + 5] = __builtin_fmaf(ps, (float)e57.x, acc[8 * k + 5]);
          acc[8 * k + 6] = __builtin_fmaf(ps, (float)e46.y, acc[8 * k + 6]);
          acc[8 * k + 7] = __builtin_fmaf(ps, (float)e57.y, acc[8 * k + 7]);
        }
      }
    }
  };
  if constexpr (TOPK) {
    if (use_list) v_pass(std::true_type{});
    else v_pass(std::false_type{});
  } else {
    v_pass(std::false_type{});
  }
#pragma unroll
  for (int e = 1; e < 32; e += 2) acc[e] *= 0.0625f;   // odd dims carried a factor 16
  // lanes of one 16-lane row that own the same dims (lane = LPT * token + j) are summed
  // with DPP rotations; each row's sums go to LDS for the output step
#pragma unroll
  for (int e = 0; e < 32; ++e) acc[e] = row_sum_stride<LPT>(acc[e]);
  pm = row_sum_stride<LPT>(pm);
  const int rw = wave * 4 + (lane >> 4);
  if ((lane & 15) < LPT) {
#pragma unroll
    for (int e = 0; e < 32; ++e) red[rw][32 * j + e] = acc[e];
    red[rw][HD + j] = pm;
  }
  __syncthreads();

  // ---- 5. output (one thread per dim): the 16 row sums in a fixed order
  if (tid < HD) {
    const int d = tid, pj = d / 32;
    float od = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) od += red[r][d] + red[r][HD + pj];
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
// block steps of a split on lanes past its end, else 1.
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
  // the longest split decides; a shorter (last) split only has more lanes past its end
  DecPlan p{nsplit, chunk, dec_unroll((std::min(chunk, T) + step - 1) / step)};
  return p;
}

// Dynamic LDS of a launch: the chunk's scores, plus the kept list for top-k.
static size_t dec_lds_bytes(int chunk, bool topk) {
  size_t b = (size_t)chunk * sizeof(float);
  if (topk) b += (size_t)chunk * sizeof(uint16_t);
  return (b + 15) / 16 * 16;
}

template <int HD, int UNR, bool TOPK>
static void launch_dec(const DecPlan& p, dim3 grid, const f16* qkv, int b0, int pos,
                       const KVViewD& v, const int32_t* pad, f16* out, float* ws,
                       float scale_log2, float sparsity, hipStream_t stream) {
  hipLaunchKernelGGL((attn_decode_kernel<HD, UNR, TOPK>), grid, dim3(256),
                     dec_lds_bytes(p.chunk, TOPK), stream, qkv, b0, pos, v, pad, p.chunk, out,
                     ws, scale_log2, sparsity);
}

template <int HD, bool TOPK>
static void launch_dec(const DecPlan& p, dim3 grid, const f16* qkv, int b0, int pos,
                       const KVViewD& v, const int32_t* pad, f16* out, float* ws,
                       float scale_log2, float sparsity, hipStream_t stream) {
  switch (p.unr) {
    case 4: launch_dec<HD, 4, TOPK>(p, grid, qkv, b0, pos, v, pad, out, ws, scale_log2, sparsity, stream); break;
    case 3: launch_dec<HD, 3, TOPK>(p, grid, qkv, b0, pos, v, pad, out, ws, scale_log2, sparsity, stream); break;
    case 2: launch_dec<HD, 2, TOPK>(p, grid, qkv, b0, pos, v, pad, out, ws, scale_log2, sparsity, stream); break;
    default: launch_dec<HD, 1, TOPK>(p, grid, qkv, b0, pos, v, pad, out, ws, scale_log2, sparsity, stream); break;
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

// Argument checks of dense decode attention (everything but the workspace).
static int check_decode_args(const uint16_t* qkv, int32_t B, int32_t b0, int32_t pos,
                             const flexq_kv4_layer* kv, const uint16_t* out) {
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
  return FLEXQ_OK;
}

// Launches the dense decode (and the merge when the context is split) with the split
// partials in ws (checked by the caller: at least the workspace size, 16-byte aligned).
static int run_decode(const uint16_t* qkv, int32_t B, int32_t b0, int32_t pos,
                      const flexq_kv4_layer* kv, uint16_t* out, void* ws, hipStream_t stream) {
  const DecPlan p = dec_plan(B, kv->heads, kv->head_dim, pos);
  KVViewD v{kv->k_codes, kv->v_codes, (uint32_t*)kv->k_params, (uint32_t*)kv->v_params, kv->heads,
            kv->max_len};
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)kv->head_dim);
  dim3 grid(p.splits, kv->heads, B);
  if (kv->head_dim == 64) {
    launch_dec<64, false>(p, grid, (const f16*)qkv, b0, pos, v, kv->pad, (f16*)out, (float*)ws,
                          scale_log2, 1.0f, stream);
    if (p.splits > 1)
      hipLaunchKernelGGL(attn_decode_merge_kernel<64>, dim3(kv->heads, B), dim3(64), 0, stream,
                         (const float*)ws, p.splits, kv->heads, (f16*)out);
  } else {
    launch_dec<128, false>(p, grid, (const f16*)qkv, b0, pos, v, kv->pad, (f16*)out,
                           (float*)ws, scale_log2, 1.0f, stream);
    if (p.splits > 1)
      hipLaunchKernelGGL(attn_decode_merge_kernel<128>, dim3(kv->heads, B), dim3(128), 0, stream,
                         (const float*)ws, p.splits, kv->heads, (f16*)out);
  }
  FLEXQ_LAUNCH_CHECK();
  return FLEXQ_OK;
}

// The split partials of flexq_attn_decode_kv4_static: a static array that every device
// the library runs on holds until the process ends.  In host code `scratch` only
// stands for the symbol; its address on a device comes from hipGetSymbolAddress, taken
// once per device with that device current and kept in scratch_ptr.
static __device__ __align__(256) float scratch[FLEXQ_STATIC_SCRATCH_BYTES / sizeof(float)];
static std::atomic<void*> scratch_ptr[kMaxDevices];

static int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FLEXQ_ERR_DEVICE;
  if (dev >= kMaxDevices) return FLEXQ_ERR_UNSUPPORTED;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return FLEXQ_ERR_DEVICE;
    }
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return FLEXQ_OK;
}

extern "C" int flexq_attn_decode_kv4(const uint16_t* qkv, int32_t B, int32_t b0, int32_t pos,
                                     const flexq_kv4_layer* kv, uint16_t* out, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  const int st = check_decode_args(qkv, B, b0, pos, kv, out);
  if (st != FLEXQ_OK || B == 0) return st;
  const size_t need = flexq_attn_decode_workspace_size(B, kv->heads, kv->head_dim, pos);
  if (need > 0 && (!ws || ws_bytes < need || ((uintptr_t)ws & 15))) return FLEXQ_ERR_INVALID;
  return run_decode(qkv, B, b0, pos, kv, out, ws, stream);
}

extern "C" int flexq_attn_decode_kv4_static(const uint16_t* qkv, int32_t B, int32_t b0,
                                            int32_t pos, const flexq_kv4_layer* kv,
                                            uint16_t* out, hipStream_t stream) {
  const int st = check_decode_args(qkv, B, b0, pos, kv, out);
  if (st != FLEXQ_OK || B == 0) return st;
  const size_t need = flexq_attn_decode_workspace_size(B, kv->heads, kv->head_dim, pos);
  if (need > FLEXQ_STATIC_SCRATCH_BYTES) return FLEXQ_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (need > 0) {
    const int sst = static_scratch(&ws);
    if (sst != FLEXQ_OK) return sst;
  }
  return run_decode(qkv, B, b0, pos, kv, out, ws, stream);
}

extern "C" int flexq_attn_decode_kv4_topk(const uint16_t* qkv, int32_t B, int32_t b0, int32_t pos,
                                          const flexq_kv4_layer* kv, float sparsity,
                                          uint16_t* out, hipStream_t stream) {
  if (!(sparsity > 0.0f) || !(sparsity <= __FLT_MAX__)) return FLEXQ_ERR_INVALID;
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
  if (pos + 1 > kDecMaxChunk) return FLEXQ_ERR_UNSUPPORTED;   // the scores live in LDS
  const int step = kv->head_dim == 128 ? 64 : 128;
  DecPlan p{1, pos + 1, dec_unroll((pos + 1 + step - 1) / step)};
  KVViewD v{kv->k_codes, kv->v_codes, (uint32_t*)kv->k_params, (uint32_t*)kv->v_params, kv->heads,
            kv->max_len};
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)kv->head_dim);
  dim3 grid(1, kv->heads, B);
  if (kv->head_dim == 64)
    launch_dec<64, true>(p, grid, (const f16*)qkv, b0, pos, v, kv->pad, (f16*)out, nullptr,
                         scale_log2, sparsity, stream);
  else
    launch_dec<128, true>(p, grid, (const f16*)qkv, b0, pos, v, kv->pad, (f16*)out, nullptr,
                          scale_log2, sparsity, stream);
  FLEXQ_LAUNCH_CHECK();
  return FLEXQ_OK;
}
