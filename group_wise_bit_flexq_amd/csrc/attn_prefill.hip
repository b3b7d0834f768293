// Prefill attention (the pages' `mha`, source notes section "Pytorch Backend") with
// the 4-bit KV store fused at the end (walkthrough section 6.3, cache config:
// group 64 along head_dim).
//
// One work-group per (128-query block, head, sequence), two resident per CU; 4 waves
// of 32 queries, one MFMA tile (v_mfma_f32_32x32x16_f16) wide.  Key blocks of 64 positions are staged
// in LDS by 16-B copies (K rows XOR-swizzled, V rows padded), two stages deep: the
// next block is loaded into registers while the current one is multiplied, one
// barrier per block.
//  * scores S^T = K . Q^T, 32 keys x 32 queries per tile: the K operand is read from
//    LDS, Q^T stays in registers; lane l owns query l % 32 and 16 keys of each tile
//    (rows 8 (r / 4) + 4 (l / 32) + r % 4), so a query's softmax statistics need
//    one exchange with lane l ^ 32;
//  * online softmax in fp32 (exp2 with 1/sqrt(hd) * log2(e) fused into its argument,
//    lazy rescaling of the output when a query's running max grows by more than 8);
//  * O^T += V^T . P^T, 16 keys per MFMA: the probabilities are used from the score
//    registers as the B operand (register r of tile t is key 32 t + 16 (r / 8) +
//    8 ((r / 4) % 2) + 4 (l / 32) + r % 4), and the matching V^T operand -- four
//    consecutive keys of one dimension per lane, twice -- comes straight from the
//    row-major V tile through the transposing LDS read ds_read_b64_tr_b16: within
//    each 16-lane group, lane j points at 4 dims of key j / 4 and lane i receives
//    dim i of the 4 keys.
// After the loop the work-group quantizes K and V of its own 128 positions into the
// cache (one lane per 64-element group), reading them from the staged LDS tiles.
// Left padding (the generation loop's attention mask): keys below the sequence's pad
// count are masked, key blocks wholly below it are skipped (except the work-group's
// own two, which the store needs staged), and a query with no visible key writes 0.
#include "host_cache.h"
#include "quant_dev.h"

namespace flexq {

struct KVView {
  uint8_t* kc;
  uint8_t* vc;
  uint32_t* kp;
  uint32_t* vp;
  int nh, max_len;
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

template <int HD>
struct PrefillShape {
  static constexpr int QB = 128;                 // queries per work-group
  static constexpr int KB = 64;                  // keys per block step
  static constexpr int HC = HD / 8;              // 16-B chunks per K/V row
  static constexpr int VLD = HD + 32;            // padded V row (halves): rows 4 apart
                                                 // in LDS banks for the transposing read
  static constexpr int K_STAGE = KB * HD;        // halves
  static constexpr int V_STAGE = KB * VLD;       // halves
  static constexpr int CH_PER_T = KB * HC / 256; // 16-B chunks of K (and of V) per thread
  static constexpr size_t LDS_BYTES = 2 * (size_t)(K_STAGE + V_STAGE) * sizeof(f16);
};

// swizzled position of 16-B chunk `ch` in K row `row` (conflict-free b128 reads of
// 32 consecutive rows at one chunk)
template <int HD>
__device__ __forceinline__ int k_off(int row, int ch) {
  if constexpr (HD == 128) return row * HD + ((ch ^ (row & 15)) << 3);
  else return row * HD + ((ch ^ ((row >> 1) & 7)) << 3);
}

// Lane l receives x of lanes l % 32 and 32 + l % 32 (v_permlane32_swap): the two
// halves of a query's statistics, in the same order on both lanes that hold them.
__device__ __forceinline__ void lane_halves(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

template <int HD>
__global__ __launch_bounds__(256, 2) void attn_prefill_kernel(const f16* __restrict__ qkv, int S,
                                                           int nh, int b0, KVView kv,
                                                           const int32_t* __restrict__ pad,
                                                           f16* __restrict__ out,
                                                           float scale_log2) {
  using P = PrefillShape<HD>;
  constexpr int QB = P::QB, KB = P::KB, HC = P::HC, VLD = P::VLD;
  constexpr int KS = HD / 16;        // k-steps of a score tile
  constexpr int DT = HD / 32;        // output dim tiles
  constexpr int CPT = P::CH_PER_T;
  extern __shared__ __attribute__((aligned(16))) f16 smem[];
  f16* const sK = smem;                          // [2][KB * HD]
  f16* const sV = smem + 2 * P::K_STAGE;         // [2][KB * VLD]

  // 1-D grid of (query block, head, sequence) items.  The dispatcher deals work-groups
  // to the 8 XCDs round-robin; item order is remapped so that each XCD runs a
  // contiguous range, in which the query blocks of one (sequence, head) -- which
  // stage the same K/V rows -- follow each other and share that XCD's L2.  Long
  // (late) query blocks come first within each (sequence, head).
  const int nqb = (S + QB - 1) / QB;
  const int items = (int)gridDim.x;
  int w = blockIdx.x;
  if (items % 8 == 0) w = (w & 7) * (items >> 3) + (w >> 3);
  const int qb = nqb - 1 - w % nqb;
  const int head = (w / nqb) % nh;
  const int b = w / (nqb * nh);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = nh * HD;
  const int64_t ld = 3 * (int64_t)h;
  const f16* base = qkv + (int64_t)b * S * ld;
  const int q0 = qb * QB;
  const int wq0 = q0 + wave * 32;          // first query of this wave
  const int hl = lane >> 5;                // lane half
  const int qabs = wq0 + (lane & 31);
  const int qrow = min(qabs, S - 1);
  const int kend = min(q0 + QB, S);        // keys this work-group needs: [pb, kend)
  const int nkb = (kend + KB - 1) / KB;
  const int pb = pad ? min(max(pad[b0 + b], 0), S - 1) : 0;
  const int kb0 = min(pb / KB, 2 * qb);    // the own blocks 2 qb, 2 qb + 1 stay staged

  // Q^T operand: lane (q, half) holds Q[q][16 ks + 8 half .. +7]
  f16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = *(const f16x8*)(base + (int64_t)qrow * ld + head * HD + 16 * ks + 8 * hl);

  f32x16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = (f32x16){0};
  float m_run = -INFINITY, l_run = 0.0f;

  // staging: thread t copies chunks c = t + 256 u of the block's K and V rows
  // (row c / HC, chunk c % HC) through a raw buffer view of the block's rows that ends
  // at key S - 1: the per-lane offsets are fixed, the block moves the view's base, and
  // keys past S read zeros (they are masked).  The registers are named scalars (arrays
  // of them would live in scratch memory).
  static_assert(CPT == 2 || CPT == 4, "staging copies are stamped out for 2 or 4 per thread");
  uint4 rk0, rk1, rk2, rk3, rv0, rv1, rv2, rv3;
  int voff0 = 0, voff1 = 0, voff2 = 0, voff3 = 0;
#define PF_OFF(u)                                                                          \
  if constexpr ((u) < CPT) {                                                               \
    const int _c = tid + 256 * (u);                                                        \
    voff##u = ((_c / HC) * (int)ld + head * HD + (_c % HC) * 8) * (int)sizeof(f16);       \
  }
  PF_OFF(0) PF_OFF(1) PF_OFF(2) PF_OFF(3)
#undef PF_OFF
#define PF_LD(u, RS_)                                                                      \
  if constexpr ((u) < CPT) {                                                               \
    rk##u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(               \
        RS_, voff##u, h * (int)sizeof(f16), 0));                                           \
    rv##u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(               \
        RS_, voff##u, 2 * h * (int)sizeof(f16), 0));                                       \
  }
#define PF_ST(u, ST_)                                                           \
  if constexpr ((u) < CPT) {                                                    \
    const int _c = tid + 256 * (u);                                             \
    const int _r = _c / HC, _ch = _c % HC;                                      \
    *(uint4*)(sK + (ST_) * P::K_STAGE + k_off<HD>(_r, _ch)) = rk##u;            \
    *(uint4*)(sV + (ST_) * P::V_STAGE + _r * VLD + _ch * 8) = rv##u;            \
  }
#define LOAD_KV(KB_)                                                                       \
  do {                                                                                     \
    const int _k0 = (KB_) * KB;                                                            \
    const rsrc_t _rs = make_rsrc(base + (int64_t)_k0 * ld, min(S - _k0, KB) * (int)ld * 2); \
    PF_LD(0, _rs) PF_LD(1, _rs) PF_LD(2, _rs) PF_LD(3, _rs)                                \
  } while (0)
#define STORE_KV(ST_) do { PF_ST(0, ST_) PF_ST(1, ST_) PF_ST(2, ST_) PF_ST(3, ST_) } while (0)

  // transposing-read lane geometry: 16-lane group a = lane / 16 covers dims
  // 16 (a % 2) .. +15 of a 32-dim tile and keys 4 (a / 2) .. +3 (+8) of a 16-key step
  const int tr_i = lane & 15;
  const int tr_key = 4 * hl + (tr_i >> 2);
  const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (tr_i & 3);

  LOAD_KV(kb0);
  for (int kb = kb0; kb < nkb; ++kb) {
    const int st = kb & 1;
    STORE_KV(st);
    if (kb + 1 < nkb) LOAD_KV(kb + 1);
    __syncthreads();
    const int k0 = kb * KB;
    // some key of the block is visible to some query of the wave
    if (k0 <= wq0 + 31 && k0 + KB > pb && wq0 + 31 >= pb) {
      const f16* sk = sK + st * P::K_STAGE;
      const f16* sv = sV + st * P::V_STAGE;
      f32x16 s[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        s[t] = (f32x16){0};
        const int krow = 32 * t + (lane & 31);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const f16x8 kf = *(const f16x8*)(sk + k_off<HD>(krow, 2 * ks + hl));
          s[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], s[t], 0, 0, 0);
        }
      }
      // mask (causal and past the end) and block max on the raw scores (the scale is
      // positive, so it commutes with the max).  Register r of tile t is key
      // k0 + 32 t + 8 (r / 4) + 4 (l / 32) + r % 4: one compare of its constant offset
      // against a per-lane limit.
      if ((k0 + KB - 1 > wq0) || (k0 + KB > S)) {
        const int lim = min(qabs, S - 1) - k0 - 4 * hl;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * t + 8 * (r >> 2) + (r & 3) > lim) s[t][r] = -INFINITY;
      }
      if (k0 < pb) {   // the block holds pad keys
        const int lo = pb - k0 - 4 * hl;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * t + 8 * (r >> 2) + (r & 3) < lo) s[t][r] = -INFINITY;
      }
      float mb = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mb = fmaxf(mb, s[t][r]);
      {
        float lo, hi;
        lane_halves(mb, lo, hi);
        mb = fmaxf(lo, hi) * scale_log2;
      }
      // Lazy rescaling: the reference point m_run only moves when the block max exceeds
      // it by more than 8 (probabilities stay <= 2^8, far inside fp16's range and at
      // the same relative precision); otherwise O and l keep their scale.
      const bool grow = mb > m_run + 8.0f;
      if (__builtin_amdgcn_ballot_w64(grow)) {   // wave-uniform branch
        const float m_new = grow ? mb : m_run;
        // m_run = -inf on the first block -> 0; lanes that keep their reference take 1
        // (also a pad query's, whose m_run stays -inf)
        const float alpha = grow ? exp2f(m_run - m_new) : 1.0f;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DT; ++i) o[i] *= alpha;
        m_run = m_new;
      }
      // a query that has seen no visible key yet (a pad query) keeps m_run = -inf:
      // its masked scores then give p = 2^-inf = 0 instead of 2^(-inf + inf)
      const float m_ref = m_run == -INFINITY ? 0.0f : m_run;
      float ls = 0.0f;
      f16x8 pf[4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // v_exp_f32: results below 2^-126 flush to 0 (they vanish in the fp16 P anyway)
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], scale_log2, -m_ref));
          ls += p;
          pf[2 * t + (r >> 3)][r & 7] = (f16)p;
        }
      {
        float lo, hi;
        lane_halves(ls, lo, hi);
        l_run += lo + hi;
      }
      // O^T += V^T P^T over the four 16-key steps
#pragma unroll
      for (int ss = 0; ss < 4; ++ss) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const f16* vp = sv + (16 * ss + tr_key) * VLD + 32 * dt + tr_dim;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vp));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vp + 8 * VLD));
          const f16x8 vf = __builtin_bit_cast(
              f16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[ss], o[dt], 0, 0, 0);
        }
      }
    }
  }

#undef PF_LD
#undef PF_ST
#undef LOAD_KV
#undef STORE_KV

  // O^T lane l reg r = dim 32 dt + 8 (r / 4) + 4 (l / 32) + r % 4 of query l % 32
  if (qabs < S) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;   // 0 for a pad query
    f16* orow = out + ((int64_t)b * S + qabs) * h + head * HD;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x4 v = (f16x4){(f16)(o[dt][4 * j] * inv), (f16)(o[dt][4 * j + 1] * inv),
                                (f16)(o[dt][4 * j + 2] * inv), (f16)(o[dt][4 * j + 3] * inv)};
        *(f16x4*)(orow + 32 * dt + 8 * j + 4 * hl) = v;
      }
  }

  // 4-bit store of K and V for positions [q0, q0 + 128) from the staged tiles (key
  // block 2 qb + i sits in stage i; the last block's stores preceded the last barrier).
  // One lane per 64-element group: thread t quantizes group t % GPT of position
  // t / GPT, first of K, then of V, so no group statistic is computed twice and no
  // lanes exchange anything; the two groups of a position sit in adjacent lanes and a
  // wave writes whole cache lines of codes.
  constexpr int GPT = HD / 64;                     // groups per token vector
  static_assert(QB * GPT <= 256, "one group per thread and pass");
  if (tid < QB * GPT) {
    const int tr = tid / GPT;                      // position within the 128
    const int grp = tid % GPT;
    const int tok = q0 + tr;
    const int stg = tr / KB, row = tr % KB;
    const int64_t slot = ((int64_t)(b0 + b) * kv.nh + head) * kv.max_len + tok;
#pragma unroll
    for (int isv = 0; isv < 2; ++isv) {
      f16x8 x[8];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        x[c] = isv ? *(const f16x8*)(sV + stg * P::V_STAGE + row * VLD + (grp * 8 + c) * 8)
                   : *(const f16x8*)(sK + stg * P::K_STAGE + k_off<HD>(row, grp * 8 + c));
      uint32_t packed[8];
      const uint32_t prm = GroupQ<1>::run(x, packed);
      if (tok < S) {
        uint4* cdst = (uint4*)((isv ? kv.vc : kv.kc) + slot * (HD / 2) + grp * 32);
        cdst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        cdst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
        (isv ? kv.vp : kv.kp)[slot * GPT + grp] = prm;
      }
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
      ((uintptr_t)kv->v_codes & 15) || ((uintptr_t)kv->k_params & 3) || ((uintptr_t)kv->v_params & 3) ||
      ((uintptr_t)kv->pad & 3))
    return FLEXQ_ERR_INVALID;
  if (kv->heads > 65535 || B > 65535) return FLEXQ_ERR_UNSUPPORTED;
  // a key block (64 rows of q, k, v) is addressed with 32-bit byte offsets
  if ((int64_t)64 * 3 * kv->heads * kv->head_dim * 2 >= ((int64_t)1 << 31)) return FLEXQ_ERR_UNSUPPORTED;
  KVView v{kv->k_codes, kv->v_codes, (uint32_t*)kv->k_params, (uint32_t*)kv->v_params, kv->heads,
           kv->max_len};
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)kv->head_dim);
  const int64_t items = (int64_t)((S + 127) / 128) * kv->heads * B;
  if (items > 0x7FFFFFFF) return FLEXQ_ERR_UNSUPPORTED;
  dim3 grid((unsigned)items);
  static PerDeviceInt attr_set;   // 72 KB of LDS for head_dim 128: above the default limit
  (void)attr_set.get([] {
    return hipFuncSetAttribute((const void*)attn_prefill_kernel<128>,
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)PrefillShape<128>::LDS_BYTES) == hipSuccess ? 1 : 0;
  }, 0);
  if (kv->head_dim == 64)
    hipLaunchKernelGGL(attn_prefill_kernel<64>, grid, dim3(256), PrefillShape<64>::LDS_BYTES, stream,
                       (const f16*)qkv, S, kv->heads, b0, v, kv->pad, (f16*)out, scale_log2);
  else
    hipLaunchKernelGGL(attn_prefill_kernel<128>, grid, dim3(256), PrefillShape<128>::LDS_BYTES,
                       stream, (const f16*)qkv, S, kv->heads, b0, v, kv->pad, (f16*)out,
                       scale_log2);
  FLEXQ_LAUNCH_CHECK();
  return FLEXQ_OK;
}
