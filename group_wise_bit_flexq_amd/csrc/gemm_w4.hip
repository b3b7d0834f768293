// Dequant-fused 4-bit-weight GEMM on gfx950 MFMA:  y = x . W^T (+ epilogue).
//
// The pages' linear layers are fp16 matmuls whose weights are stored compressed
// (FlexGen walkthrough, section 6.3: weights grouped along the input dimension,
// 64 per group, 4 bits, fp16 parameters).  Three kernels share the arithmetic:
//
//  * large M (prefill, M = 48 x 512): 256 x 256 x 64 tiles, 8 waves.  The weight
//    tile is expanded to fp16 on its way into LDS (v_pk_fma_f16: one rounding of
//    c * scale + offset), once per work-group and k-step, and reused by all 256 rows;
//  * decode batches (64 < M <= 144): every operand goes straight from memory into a
//    5-stage LDS ring (buffer loads with the LDS flag); each wave expands only its
//    own weight columns, in registers, so every weight is read and expanded once;
//  * other small M (M <= 64, 144 < M <= 160): weight codes are streamed straight
//    into the registers of the wave that uses them and expanded there; only the
//    activation tile goes through LDS.
//
// All feed the matrix cores with fp16 operands and fp32 accumulators and finish with
// a fused bias / ReLU / residual epilogue and a single fp16 rounding.  Where a shape
// has too few tiles for the CUs, K is split and a second kernel adds the fp32 partial
// sums in split order (deterministic).
#include "common.h"

namespace flexq {

constexpr int kBK = 64;

// LDS tile rows are 128 B (8 chunks of 16 B).  gfx950's LDS serves 16 lanes of a
// 128-bit access per cycle from 64 banks, i.e. 16 slots of 16 B, and slot =
// 8 * (row & 1) + chunk for an unswizzled tile; storing chunk c of row r at chunk
// c ^ ((r >> 1) & 7) gives 16 consecutive rows read at one k offset 16 distinct
// slots, and keeps the row-wise stores conflict-free as well.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kBK + ((chunk ^ ((row >> 1) & 7)) << 3);  // in fp16 elements
}

enum OutKind { kOutF16 = 0, kOutF32 = 1, kOutPartial = 2 };

template <int WM, int WN, int TM, int TN>
struct GemmShape {
  static constexpr int BM = WM * TM * 32;
  static constexpr int BN = WN * TN * 32;
  static constexpr int THREADS = WM * WN * 64;
  static constexpr int A_CHUNKS = BM * 8;      // 16-B pieces of an A tile
  static constexpr int B_PIECES = BN * 2;      // 16-B code pieces (32 codes) of a B tile
  static constexpr int A_PER_T = (A_CHUNKS + THREADS - 1) / THREADS;
  static constexpr int B_PER_T = (B_PIECES + THREADS - 1) / THREADS;
  static constexpr size_t LDS_BYTES = 2 * (size_t)(BM + BN) * kBK * sizeof(f16);
};

struct Epilogue {
  const f16* bias;      // [N] or null
  const f16* residual;  // [M][N] or null
  int relu;
};

__device__ __forceinline__ float epilogue_value(float v, const Epilogue& ep, int64_t row, int col,
                                                int N) {
  if (ep.bias) v += (float)ep.bias[col];
  if (ep.relu) v = fmaxf(v, 0.0f);
  if (ep.residual) v += (float)ep.residual[row * N + col];
  return v;
}

// Store one 32 x 32 MFMA accumulator tile: lane l holds column `col` and rows
// row0 + 8 (r / 4) + 4 (l / 32) + r % 4, r = 0..15.  Tiles whose rows all lie below M
// take a branch-free path, so the bias and the 16 residual loads are issued together
// instead of one dependent load per element.
template <int OUT>
__device__ __forceinline__ void store_acc_tile(const f32x16& a, int row0, int col, int M, int N,
                                               const Epilogue& ep, void* __restrict__ Y,
                                               int split) {
  const int rl = row0 + 4 * ((threadIdx.x & 63) >> 5);
  if (row0 + 32 <= M) {
    if (col >= N) return;
    if constexpr (OUT == kOutF16) {
      const float b = ep.bias ? (float)ep.bias[col] : 0.0f;
      float res[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) res[r] = 0.0f;
      if (ep.residual) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          res[r] = (float)ep.residual[(int64_t)(rl + 8 * (r >> 2) + (r & 3)) * N + col];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = a[r] + b;
        if (ep.relu) v = fmaxf(v, 0.0f);
        v += res[r];
        ((f16*)Y)[(int64_t)(rl + 8 * (r >> 2) + (r & 3)) * N + col] = (f16)v;
      }
    } else {
      float* const y = (float*)Y + (OUT == kOutPartial ? (int64_t)split * M * N : 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) y[(int64_t)(rl + 8 * (r >> 2) + (r & 3)) * N + col] = a[r];
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = rl + 8 * (r >> 2) + (r & 3);
    if (row < M && col < N) {
      if constexpr (OUT == kOutF16) {
        ((f16*)Y)[(int64_t)row * N + col] = (f16)epilogue_value(a[r], ep, row, col, N);
      } else {
        float* const y = (float*)Y + (OUT == kOutPartial ? (int64_t)split * M * N : 0);
        y[(int64_t)row * N + col] = a[r];
      }
    }
  }
}

// ------------------------------------------------------------------ large-M kernel
//
// Prefill shapes (M = 48 x 512 rows) use a 256 x 256 x 64 tile with 8 waves
// (2 x 4, 128 x 64 each) and a software pipeline that keeps the matrix cores fed:
// while the MFMAs of k-tile kt run from LDS stage kt % 2, the same waves write
// k-tile kt+1 (already in registers) into the other stage -- A tile copied, W tile
// dequantized on the way -- and issue the global loads of k-tile kt+2.  One barrier
// per k-tile.  On gfx950 independent VALU work only partly overlaps a running MFMA
// and LDS writes are about 2.5x slower per byte than reads, so the loop is ordered by
// hand: every MFMA is followed by a small pinned slice of the side work.
//
// Tile order: the dispatcher deals work-groups to the 8 XCDs round-robin, so XCD x
// runs work-groups x, x + 8, ...  XCD x is given the N-tile range [x nx, (x+1) nx)
// and walks it in groups of 4 M-tiles; at any moment all XCDs work on the same 4
// M-tiles, whose A rows are then shared through the last-level cache instead of
// being fetched from HBM by each XCD, and the ~32 tiles resident on one XCD form a
// 4 x 8 block whose A rows (32 KB per k-tile each) and W columns (9 KB) its L2
// shares -- the shape with the fewest L2 misses for those sizes.
__device__ __forceinline__ void big_tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int G = 4;
  const int bid = blockIdx.x;
  if (tiles_n % 8 == 0) {
    const int x = bid & 7, q = bid >> 3, nx = tiles_n >> 3;
    const int per_group = G * nx;
    const int group = q / per_group;
    const int first_m = group * G;
    const int gsize = min(tiles_m - first_m, G);
    const int r = q - group * per_group;
    tm = first_m + r % gsize;
    tn = x * nx + r / gsize;
    return;
  }
  // other widths: plain groups of 4 M-tiles in launch order
  const int per_group = G * tiles_n;
  const int group = bid / per_group;
  const int first_m = group * G;
  const int gsize = min(tiles_m - first_m, G);
  const int r = bid - group * per_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

template <int WM, int WN, int TM, int TN, int OUT>
__global__ __launch_bounds__(WM* WN * 64, 1) void gemm_w4_big_kernel(
    const f16* __restrict__ X, const uint8_t* __restrict__ Wc, const uint32_t* __restrict__ Wp,
    int M, int N, int K, int kt_per_split, Epilogue ep, void* __restrict__ Y) {
  using S = GemmShape<WM, WN, TM, TN>;
  constexpr int AJ = S::A_PER_T;           // 16-B A chunks per thread and k-tile
  constexpr int BJ = S::B_PER_T;           // 16-B W code pieces per thread and k-tile
  constexpr int AROWS = S::THREADS / 8;    // rows covered by one pass of A loads
  static_assert(S::A_CHUNKS % S::THREADS == 0 && S::B_PIECES % S::THREADS == 0, "tile split");
  extern __shared__ __attribute__((aligned(16))) f16 smem[];
  f16* const sA = smem;                       // [2][BM*64]
  f16* const sB = smem + 2 * S::BM * kBK;     // [2][BN*64]
  constexpr int kStageA = S::BM * kBK, kStageB = S::BN * kBK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  int tm, tn;
  big_tile_coords((M + S::BM - 1) / S::BM, (N + S::BN - 1) / S::BN, tm, tn);
  const int m0 = tm * S::BM, n0 = tn * S::BN;
  const int KT = K / kBK;
  const int kt0 = blockIdx.y * kt_per_split;
  const int kt1 = min(KT, kt0 + kt_per_split);

  // The k-loop below is written out by hand for the 256 x 256 tile of 8 waves (2 x 4),
  // each wave owning 128 x 64 outputs as 4 x 2 MFMA tiles of 32 x 32.
  static_assert(WM == 2 && WN == 4 && TM == 4 && TN == 2, "k-loop is written for this tile");
  static_assert(AJ == 4 && BJ == 1, "per-thread share of the A and B tiles");

  // A: thread t copies chunk (t & 7) of tile rows (t >> 3) + 64 j, j = 0..3.  Rows past M
  // read the tile's first row instead and are never stored, so every load stays in
  // bounds without a branch; the same holds for W rows past N.  Per-thread state lives
  // in named scalars: the compiler puts arrays of them in scratch memory.
  const int a_row = tid >> 3, a_ch = tid & 7;
#define A_SRC(j)                                                                         \
  const f16* const a_src##j =                                                            \
      X + (int64_t)(m0 + a_row + AROWS * j < M ? m0 + a_row + AROWS * j : m0) * K + a_ch * 8;
  A_SRC(0) A_SRC(1) A_SRC(2) A_SRC(3)
#undef A_SRC
  // lds_off(row + 64 j, ch) = lds_off(row, ch) + 64 j * 64 (the swizzle sees row bits 1-3)
  const int a_lds = lds_off(a_row, a_ch);
  // B: thread t expands the 32 codes of W row t >> 1, half t & 1 of the 64-code group:
  // word q of its 16-B piece becomes LDS chunk 4 (t & 1) + q of that row.
  const int b_row = tid >> 1, b_half = tid & 1;
  const int b_gn = n0 + b_row < N ? n0 + b_row : n0;
  const uint8_t* const b_src = Wc + w4_code_off(b_gn, 0, KT) + b_half * 16;
  const uint32_t* const p_src = Wp + w4_param_idx(b_gn, 0, KT);
  const int b_lds0 = lds_off(b_row, b_half * 4 + 0), b_lds1 = lds_off(b_row, b_half * 4 + 1);
  const int b_lds2 = lds_off(b_row, b_half * 4 + 2), b_lds3 = lds_off(b_row, b_half * 4 + 3);
  uint4 ra0, ra1, ra2, ra3;         // A chunks of the next k-tile
  uint4 rb_0, rb_1;                 // W codes, two k-tiles in flight (set = tile parity)
  uint32_t rp_0, rp_1;              // their (offset, step) words
  uint32_t dq_t0, dq_t1, dq0, dq1, dq2, dq3;
  f16x2 dq_s, dq_m;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){0};
  // fragment sets: k-steps alternate between set 0 and set 1
  f16x8 fa0[TM], fb0[TN], fa1[TM], fb1[TN];

  // Lane (l & 31) of a fragment is row (l & 31) of its 32-row slice; lane half l >> 5
  // takes k 8 (l >> 5) .. +8 of the 16-wide k-step, i.e. LDS chunk 2 ks + (l >> 5).
  // The swizzle term (row >> 1) & 7 is the same for every 32-row slice of the wave.
  const int fa_row = wm * TM * 32 + (lane & 31), fb_row = wn * TN * 32 + (lane & 31);
  const int fa_base = fa_row * 64, fb_base = fb_row * 64;
  const int f_sw = (fa_row >> 1) & 7;    // == (fb_row >> 1) & 7: both rows are lane & 31 + 32 x
  const int f_ch = lane >> 5;

#define SB() __builtin_amdgcn_sched_barrier(0)
#define MF(FA, FB, i, j) \
  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(FA[i], FB[j], acc[i][j], 0, 0, 0)
#define FRAG_A(F, BUF, KS, i) \
  F[i] = *(const f16x8*)(sA + (BUF) * kStageA + fa_base + (i) * 32 * 64 + (((2 * (KS) + f_ch) ^ f_sw) << 3))
#define FRAG_B(F, BUF, KS, j) \
  F[j] = *(const f16x8*)(sB + (BUF) * kStageB + fb_base + (j) * 32 * 64 + (((2 * (KS) + f_ch) ^ f_sw) << 3))
#define LOAD_A(j, KT) ra##j = *(const uint4*)(a_src##j + (int64_t)(KT) * kBK)
#define STORE_A(j, BUF) *(uint4*)(sA + (BUF) * kStageA + a_lds + AROWS * 64 * j) = ra##j
#define LOAD_B(SET, KT)                                   \
  do {                                                    \
    rb_##SET = *(const uint4*)(b_src + (int64_t)(KT) * kW4TileBytes); \
    rp_##SET = p_src[(int64_t)(KT) * kW4BlockRows];                   \
  } while (0)
#define DQ_SCALE(SET)                                     \
  do {                                                    \
    dq_s = h2_from_u32((rp_##SET >> 16) * 0x10001u);      \
    dq_m = h2_from_u32((rp_##SET & 0xFFFFu) * 0x10001u);  \
  } while (0)
#define DQ_PRE(W) w4_word_to_bytes((W), dq_t0, dq_t1)
// pair p of the word: elements 2p and 2p + 1
#define DQ_PAIR(p) \
  dq##p = u32_from_h2(dequant_pair(code_pair_f16<(p) & 1>((p) < 2 ? dq_t0 : dq_t1), dq_s, dq_m))
#define STORE_B(q, BUF) *(uint4*)(sB + (BUF) * kStageB + b_lds##q) = make_uint4(dq0, dq1, dq2, dq3)

// One k-step region: the 8 MFMAs of fragment set (FA, FB), each followed by a pinned
// slice of side work so that the matrix core always has the next MFMA queued while
// the wave issues VALU, LDS and global work: the 6 fragment reads of the next k-step
// (set NA, NB, k-step KS of stage BUF), one A chunk of k-tile kt+1 (LDS stage NBUF),
// one W word of it dequantized into stage NBUF, and the global load of A chunk R of
// k-tile kt+2 (K2).  Region 0 also loads the W codes of k-tile kt+2 (set LSET) and
// takes the scale of k-tile kt+1 (set USET).
#define REGION(FA, FB, NA, NB, BUF, KS, R, WORD, NBUF, USET, LSET, K2) \
  do {                                                                 \
    MF(FA, FB, 0, 0); SB();                                            \
    FRAG_A(NA, BUF, KS, 0); FRAG_B(NB, BUF, KS, 0); SB();              \
    MF(FA, FB, 0, 1); SB();                                            \
    FRAG_B(NB, BUF, KS, 1); STORE_A(R, NBUF); SB();                    \
    MF(FA, FB, 1, 0); SB();                                            \
    FRAG_A(NA, BUF, KS, 1); LOAD_A(R, K2);                             \
    if ((R) == 0) { DQ_SCALE(USET); LOAD_B(LSET, K2); }                \
    SB();                                                              \
    MF(FA, FB, 1, 1); SB();                                            \
    FRAG_A(NA, BUF, KS, 2); DQ_PRE(rb_##USET.WORD); DQ_PAIR(0); SB();  \
    MF(FA, FB, 2, 0); SB();                                            \
    FRAG_A(NA, BUF, KS, 3); DQ_PAIR(1); SB();                          \
    MF(FA, FB, 2, 1); SB();                                            \
    DQ_PAIR(2); SB();                                                  \
    MF(FA, FB, 3, 0); SB();                                            \
    DQ_PAIR(3); STORE_B(R, NBUF); SB();                                \
    MF(FA, FB, 3, 1); SB();                                            \
  } while (0)
// One k-tile kt in LDS stage BUF (k-tile kt+1 goes to the other stage); region 0
// finishes the previous k-tile's last k-step (all-zero fragments before the first).
#define TILE(BUF, NBUF, KT)                                                           \
  do {                                                                                \
    const int _k2 = min((KT) + 2, klast);                                             \
    REGION(fa1, fb1, fa0, fb0, BUF, 0, 0, x, NBUF, NBUF, BUF, _k2);                   \
    REGION(fa0, fb0, fa1, fb1, BUF, 1, 1, y, NBUF, NBUF, BUF, _k2);                   \
    REGION(fa1, fb1, fa0, fb0, BUF, 2, 2, z, NBUF, NBUF, BUF, _k2);                   \
    REGION(fa0, fb0, fa1, fb1, BUF, 3, 3, w, NBUF, NBUF, BUF, _k2);                   \
    __syncthreads();                                                                  \
  } while (0)

  // Software pipeline over k-tiles.  While k-tile kt is multiplied out of LDS stage
  // (kt - kt0) & 1, the same waves write k-tile kt+1 (registers -> the other stage, W
  // dequantized on the way) and issue the global loads of k-tile kt+2; the k-steps are
  // rotated by one so that MFMAs follow each barrier at once.  Loads and stores are
  // unconditional (indices clamped to the last k-tile), which keeps the counts of
  // outstanding loads exact; the final stores fill a stage no one reads.  The loop is
  // unrolled by two so that stage offsets are constants.
  if (kt0 < kt1) {
    const int klast = kt1 - 1;
    const int k1 = min(kt0 + 1, klast);
    LOAD_A(0, kt0); LOAD_A(1, kt0); LOAD_A(2, kt0); LOAD_A(3, kt0);
    LOAD_B(0, kt0);
    STORE_A(0, 0); STORE_A(1, 0); STORE_A(2, 0); STORE_A(3, 0);
    DQ_SCALE(0);
    DQ_PRE(rb_0.x); DQ_PAIR(0); DQ_PAIR(1); DQ_PAIR(2); DQ_PAIR(3); STORE_B(0, 0);
    DQ_PRE(rb_0.y); DQ_PAIR(0); DQ_PAIR(1); DQ_PAIR(2); DQ_PAIR(3); STORE_B(1, 0);
    DQ_PRE(rb_0.z); DQ_PAIR(0); DQ_PAIR(1); DQ_PAIR(2); DQ_PAIR(3); STORE_B(2, 0);
    DQ_PRE(rb_0.w); DQ_PAIR(0); DQ_PAIR(1); DQ_PAIR(2); DQ_PAIR(3); STORE_B(3, 0);
    LOAD_A(0, k1); LOAD_A(1, k1); LOAD_A(2, k1); LOAD_A(3, k1);
    LOAD_B(1, k1);
#pragma unroll
    for (int i = 0; i < TM; ++i) fa1[i] = (f16x8){0};
#pragma unroll
    for (int j = 0; j < TN; ++j) fb1[j] = (f16x8){0};
    __syncthreads();
    int kt = kt0;
    for (; kt + 1 < kt1; kt += 2) {
      TILE(0, 1, kt);
      TILE(1, 0, kt + 1);
    }
    if (kt < kt1) TILE(0, 1, kt);
    _Pragma("unroll") for (int i = 0; i < TM; ++i)
        _Pragma("unroll") for (int j = 0; j < TN; ++j) MF(fa1, fb1, i, j);
  }
#undef SB
#undef MF
#undef FRAG_A
#undef FRAG_B
#undef LOAD_A
#undef STORE_A
#undef LOAD_B
#undef DQ_SCALE
#undef DQ_PRE
#undef DQ_PAIR
#undef STORE_B
#undef REGION
#undef TILE

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
      store_acc_tile<OUT>(acc[i][j], m0 + wm * TM * 32 + i * 32,
                          n0 + wn * TN * 32 + j * 32 + (lane & 31), M, N, ep, Y, blockIdx.y);
}

// ------------------------------------------------------------------ small-M kernel
//
// Decode shapes (M <= 160 rows: the whole batch of one step) are weight-streaming:
// every W element is used by exactly one wave, so W never goes through LDS.  Each
// wave owns TN x 32 output columns and loads its own codes straight into registers,
// two k-tiles ahead; only the activation tile (M x 64) is staged in LDS and shared.
// The k index inside a 64-wide k-tile is permuted so that one 16-B code load per
// lane is exactly its MFMA B operand for all four k-steps: in k-step ks, lane l
// (lane group g = l / 32) holds k = 32 g + 8 ks + e, e = 0..7.  The A operand is
// read from LDS with the same numbering (chunk 4 g + ks of the row), so every
// product pairs matching k.
template <int MT, int NW, int TN>
struct SkinnyShape {
  static constexpr int BM = MT * 32;
  static constexpr int BN = NW * TN * 32;
  static constexpr int THREADS = NW * 64;
  static constexpr int A_CHUNKS = BM * 8;
  static constexpr int A_PER_T = (A_CHUNKS + THREADS - 1) / THREADS;
  static constexpr size_t LDS_BYTES = 2 * (size_t)BM * kBK * sizeof(f16);
};

template <int MT, int NW, int TN, int OUT>
__global__ __launch_bounds__(NW * 64) void gemm_w4_skinny_kernel(
    const f16* __restrict__ X, const uint8_t* __restrict__ Wc, const uint32_t* __restrict__ Wp,
    int M, int N, int K, int kt_per_split, Epilogue ep, void* __restrict__ Y) {
  using S = SkinnyShape<MT, NW, TN>;
  static_assert(NW == 4 && TN == 2 && MT >= 1 && MT <= 5, "k-loop is written for 4 waves x 64 columns");
  static_assert(S::A_CHUNKS == MT * S::THREADS, "one A chunk per thread and 32 rows");
  extern __shared__ __attribute__((aligned(16))) f16 smem[];
  constexpr int kStageA = S::BM * kBK;
  constexpr int NS = MT * TN;             // MFMAs (= side-work slices) per k-step

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int n0 = blockIdx.x * S::BN;
  const int m0 = blockIdx.z * S::BM;
  const int KT = K / kBK;
  const int kt0 = blockIdx.y * kt_per_split;
  const int kt1 = min(KT, kt0 + kt_per_split);

  // A: thread t copies chunk (t & 7) of tile rows (t >> 3) + 32 j, j < MT.  Rows past M
  // read row m0 and are never stored.
  const int a_row = tid >> 3, a_ch = tid & 7;
#define A_SRC(j)                                                                        \
  const f16* const a_src##j =                                                           \
      X + (int64_t)(m0 + a_row + 32 * (j) < M ? m0 + a_row + 32 * (j) : m0) * K + a_ch * 8;
  A_SRC(0) A_SRC(1) A_SRC(2) A_SRC(3) A_SRC(4)
#undef A_SRC
  const int a_lds = lds_off(a_row, a_ch);   // + 32 j * 64 for row + 32 j
  // A chunks of two k-tiles in flight: set = (k-tile - kt0) & 1, the LDS stage it goes to
  uint4 ra0_0, ra0_1, ra0_2, ra0_3, ra0_4, ra1_0, ra1_1, ra1_2, ra1_3, ra1_4;
  // B: lane l of wave w reads 16 B (32 codes, k = 32 g .. 32 g + 31 of the k-tile) of
  // W row n0 + (2 w + j) 32 + l % 32, and that row's (offset, scale) word.
  const int b_n0 = n0 + wave * 64 + (lane & 31), b_n1 = b_n0 + 32;
  const int b_g0 = b_n0 < N ? b_n0 : 0, b_g1 = b_n1 < N ? b_n1 : 0;
  const uint8_t* const b_src0 = Wc + w4_code_off(b_g0, 0, KT) + g * 16;
  const uint8_t* const b_src1 = Wc + w4_code_off(b_g1, 0, KT) + g * 16;
  const uint32_t* const p_src0 = Wp + w4_param_idx(b_g0, 0, KT);
  const uint32_t* const p_src1 = Wp + w4_param_idx(b_g1, 0, KT);
  // W codes of four k-tiles in flight: set = (k-tile - kt0) mod 4
  uint4 rb0_0, rb1_0, rb0_1, rb1_1, rb0_2, rb1_2, rb0_3, rb1_3;
  uint32_t rp0_0, rp1_0, rp0_1, rp1_1, rp0_2, rp1_2, rp0_3, rp1_3;
  uint32_t dq_t0, dq_t1;
  f16x2 dq_s0, dq_m0, dq_s1, dq_m1;

  f32x16 acc[MT][TN];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){0};
  f16x8 fa0[MT], fb0[TN], fa1[MT], fb1[TN];
  // A fragment of row slice i, k-step ks: LDS chunk 4 g + ks of row 32 i + (l & 31)
  const int fa_base = (lane & 31) * 64;
  const int f_sw = ((lane & 31) >> 1) & 7;

#define SB() __builtin_amdgcn_sched_barrier(0)
#define FRAG_A(F, BUF, KS, i) \
  F[i] = *(const f16x8*)(smem + (BUF) * kStageA + fa_base + (i) * 32 * 64 + (((4 * g + (KS)) ^ f_sw) << 3))
#define LOAD_A(j, SET, KT) \
  if constexpr ((j) < MT) ra##SET##_##j = *(const uint4*)(a_src##j + (int64_t)(KT) * kBK)
#define STORE_A(j, BUF) \
  if constexpr ((j) < MT) *(uint4*)(smem + (BUF) * kStageA + a_lds + 32 * 64 * (j)) = ra##BUF##_##j
#define LOAD_B(SET, KT)                                       \
  do {                                                        \
    rb0_##SET = *(const uint4*)(b_src0 + (int64_t)(KT) * kW4TileBytes); \
    rb1_##SET = *(const uint4*)(b_src1 + (int64_t)(KT) * kW4TileBytes); \
    rp0_##SET = p_src0[(int64_t)(KT) * kW4BlockRows];                   \
    rp1_##SET = p_src1[(int64_t)(KT) * kW4BlockRows];                   \
  } while (0)
#define DQ_SCALE(SET)                                         \
  do {                                                        \
    dq_s0 = h2_from_u32((rp0_##SET >> 16) * 0x10001u);        \
    dq_m0 = h2_from_u32((rp0_##SET & 0xFFFFu) * 0x10001u);    \
    dq_s1 = h2_from_u32((rp1_##SET >> 16) * 0x10001u);        \
    dq_m1 = h2_from_u32((rp1_##SET & 0xFFFFu) * 0x10001u);    \
  } while (0)
#define DQ_PRE(W) w4_word_to_bytes((W), dq_t0, dq_t1)
// elements 2p, 2p + 1 of B fragment F[j]
#define DQ_PAIR(F, j, p)                                                                   \
  do {                                                                                     \
    const f16x2 _d =                                                                       \
        dequant_pair(code_pair_f16<(p) & 1>((p) < 2 ? dq_t0 : dq_t1), dq_s##j, dq_m##j);   \
    F[j][2 * (p)] = _d[0];                                                                 \
    F[j][2 * (p) + 1] = _d[1];                                                             \
  } while (0)
#define MF(FA, FB, e) \
  acc[(e) / TN][(e) % TN] = __builtin_amdgcn_mfma_f32_32x32x16_f16(FA[(e) / TN], FB[(e) % TN], acc[(e) / TN][(e) % TN], 0, 0, 0)
// dequant item q (0..7) of the next k-step goes after MFMA slot q * NS / 8
#define DQ_AT(e, q) ((e) == ((q) * NS) / 8)

// One k-step region: the NS MFMAs of fragment set (FA, FB), each followed by a pinned
// slice of side work: the next k-step's A fragments (set NA, stage BUF, k-step KS)
// and B fragments (set NB, dequantized from word WORD of code set SET), A chunks of
// k-tile kt+1 stored from register set NBUF to stage NBUF and that set reloaded with
// k-tile kt+3 (chunk R, and R + 4 in region 0); region 0 also takes the scales of
// k-tile kt and loads the codes of kt+3 into set LSET.
#define REGION(FA, FB, NA, NB, BUF, KS, R, WORD, NBUF, SET, LSET, K3)     \
  do {                                                                   \
    _Pragma("unroll") for (int _e = 0; _e < NS; ++_e) {                  \
      MF(FA, FB, _e);                                                    \
      SB();                                                              \
      if (_e < MT) FRAG_A(NA, BUF, KS, _e);                              \
      if (_e == 0 && (R) == 0) { DQ_SCALE(SET); LOAD_B(LSET, K3); }      \
      if (DQ_AT(_e, 0)) { DQ_PRE(rb0_##SET.WORD); DQ_PAIR(NB, 0, 0); }   \
      if (DQ_AT(_e, 1)) DQ_PAIR(NB, 0, 1);                               \
      if (DQ_AT(_e, 2)) DQ_PAIR(NB, 0, 2);                               \
      if (DQ_AT(_e, 3)) DQ_PAIR(NB, 0, 3);                               \
      if (DQ_AT(_e, 4)) { DQ_PRE(rb1_##SET.WORD); DQ_PAIR(NB, 1, 0); }   \
      if (DQ_AT(_e, 5)) DQ_PAIR(NB, 1, 1);                               \
      if (DQ_AT(_e, 6)) DQ_PAIR(NB, 1, 2);                               \
      if (DQ_AT(_e, 7)) DQ_PAIR(NB, 1, 3);                               \
      if (_e == NS - 1) {                                                \
        STORE_A(R, NBUF); LOAD_A(R, NBUF, K3);                           \
        if ((R) == 0) { STORE_A(4, NBUF); LOAD_A(4, NBUF, K3); }         \
      }                                                                  \
      SB();                                                              \
    }                                                                    \
  } while (0)
#define TILE(BUF, NBUF, SET, LSET, KT)                                                  \
  do {                                                                                  \
    const int _k3 = min((KT) + 3, klast);                                               \
    REGION(fa1, fb1, fa0, fb0, BUF, 0, 0, x, NBUF, SET, LSET, _k3);                     \
    REGION(fa0, fb0, fa1, fb1, BUF, 1, 1, y, NBUF, SET, LSET, _k3);                     \
    REGION(fa1, fb1, fa0, fb0, BUF, 2, 2, z, NBUF, SET, LSET, _k3);                     \
    REGION(fa0, fb0, fa1, fb1, BUF, 3, 3, w, NBUF, SET, LSET, _k3);                     \
    __syncthreads();                                                                    \
  } while (0)

  // Pipeline over k-tiles (indices clamped to the last k-tile, so every load and
  // store is unconditional): while k-tile kt is multiplied out of LDS stage
  // (kt - kt0) & 1 and code set (kt - kt0) & 3, A of kt+1 is written to the other
  // stage, A and the codes of kt+3 are loaded: about 60 KB per CU in flight, enough to
  // cover HBM latency with one block per CU (vector-memory waits count loads in issue
  // order, so A and W must both be this far ahead).  The k-steps are rotated by one
  // (region 0 finishes the previous k-tile; all-zero fragments before the first), and
  // the loop is unrolled by four so that stages and code sets have fixed names.
  if (kt0 < kt1) {
    const int klast = kt1 - 1;
    const int k1 = min(kt0 + 1, klast);
    const int k2 = min(kt0 + 2, klast);
    LOAD_A(0, 0, kt0); LOAD_A(1, 0, kt0); LOAD_A(2, 0, kt0); LOAD_A(3, 0, kt0); LOAD_A(4, 0, kt0);
    LOAD_B(0, kt0);
    LOAD_A(0, 1, k1); LOAD_A(1, 1, k1); LOAD_A(2, 1, k1); LOAD_A(3, 1, k1); LOAD_A(4, 1, k1);
    LOAD_B(1, k1);
    LOAD_B(2, k2);
    STORE_A(0, 0); STORE_A(1, 0); STORE_A(2, 0); STORE_A(3, 0); STORE_A(4, 0);
    LOAD_A(0, 0, k2); LOAD_A(1, 0, k2); LOAD_A(2, 0, k2); LOAD_A(3, 0, k2); LOAD_A(4, 0, k2);
#pragma unroll
    for (int i = 0; i < MT; ++i) fa1[i] = (f16x8){0};
#pragma unroll
    for (int j = 0; j < TN; ++j) fb1[j] = (f16x8){0};
    __syncthreads();
    int kt = kt0;
    for (; kt + 3 < kt1; kt += 4) {
      TILE(0, 1, 0, 3, kt);
      TILE(1, 0, 1, 0, kt + 1);
      TILE(0, 1, 2, 1, kt + 2);
      TILE(1, 0, 3, 2, kt + 3);
    }
    if (kt < kt1) TILE(0, 1, 0, 3, kt);
    if (kt + 1 < kt1) TILE(1, 0, 1, 0, kt + 1);
    if (kt + 2 < kt1) TILE(0, 1, 2, 1, kt + 2);
#pragma unroll
    for (int e = 0; e < NS; ++e) MF(fa1, fb1, e);
  }
#undef SB
#undef FRAG_A
#undef LOAD_A
#undef STORE_A
#undef LOAD_B
#undef DQ_SCALE
#undef DQ_PRE
#undef DQ_PAIR
#undef MF
#undef DQ_AT
#undef REGION
#undef TILE

#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
      store_acc_tile<OUT>(acc[i][j], m0 + i * 32, n0 + (wave * TN + j) * 32 + (lane & 31), M, N,
                          ep, Y, blockIdx.y);
}

// ------------------------------------------------------------------ decode kernel
//
// 64 < M <= 144 (the batch of a decode step).  At these sizes the product is bound
// by streaming W, not by the matrix cores, and what limits the stream is how many
// bytes are in flight per CU: with codes staged through registers only about one
// k-tile fits, and vector loads complete in order, so the activation loads pin the
// codes' lookahead too.  Here every operand goes straight from memory to LDS
// (buffer loads with the LDS flag, no registers) through NST = 5 stages: the loads of
// k-tile kt+4 are issued while kt is computed, three k-tiles of latency are hidden and
// ~40 KB of W per CU is in flight.
//
// Stage layout: A [BM][64] fp16 with 16-byte chunk c of row r at position
// c ^ ((r >> 1) & 7) (the swizzle is applied to the source addresses, since a direct
// load writes lane i at base + 16 i); codes [384][32 B]; params [384] (offset, scale).
// 16-row MFMA tiles (v_mfma_f32_16x16x32_f16), so M = 144 needs no padding: 8 waves
// share the activation tile, each owns 48 columns (3 tiles of 16), a work-group
// covers 384 columns.  In k-step s (32 wide) lane l (group g = l / 16) holds
// k = 32 s + 8 g + e, e = 0..7: the code word at byte 16 s + 4 g of its row, and A chunk
// 4 s + g (a k-step's 64 lanes read 16 rows x 4 consecutive chunks, which with the row
// swizzle spreads over all banks: ~215 B/clk per CU against ~120 for chunks 2 g + s).  The B fragments of k-step 1 are dequantized during k-step 0, those
// of the next k-tile's k-step 0 during k-step 1 (from the next stage, which the wait
// at the top of the k-tile covers).
template <int MT16>
struct DecShape {
  static constexpr int BM = MT16 * 16;
  static constexpr int BN = 384;
  static constexpr int THREADS = 512;
  static constexpr int NST = 5;
  static constexpr int A_BYTES = BM * kBK * 2;
  static constexpr int C_BYTES = BN * 32;
  static constexpr int P_BYTES = BN * 4;
  static constexpr int STAGE_BYTES = A_BYTES + C_BYTES + P_BYTES;
  static constexpr int A_INSTR = A_BYTES / 1024;   // 16-byte loads: 1 KB per wave instruction
  static constexpr int C_INSTR = C_BYTES / 1024;
  static constexpr int P_INSTR = P_BYTES / 256;    // 4-byte loads: 256 B per wave instruction
  // every wave issues 4 sixteen-byte loads (A, else codes) and 1 four-byte load (params)
  // per stage, so all waves count the same and the waits are compile-time constants
  static constexpr int SLOTS = 5;
  static_assert(A_INSTR + C_INSTR <= 32 && P_INSTR <= 8, "loads must fit the 5 slots of 8 waves");
  static_assert(NST * STAGE_BYTES <= 160 * 1024, "stages must fit in LDS");
};

// Store one 16 x 16 MFMA accumulator tile: lane l holds column `col` and rows
// row0 + 4 (l / 16) + r, r = 0..3.
template <int OUT>
__device__ __forceinline__ void store_acc16(const f32x4& a, int row0, int col, int M, int N,
                                            const Epilogue& ep, void* __restrict__ Y,
                                            int split) {
  const int rl = row0 + 4 * ((threadIdx.x & 63) >> 4);
  if (col >= N) return;
  if constexpr (OUT == kOutF16) {
    const float b = ep.bias ? (float)ep.bias[col] : 0.0f;
    float res[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (ep.residual) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (rl + r < M) res[r] = (float)ep.residual[(int64_t)(rl + r) * N + col];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (rl + r >= M) continue;
      float v = a[r] + b;
      if (ep.relu) v = fmaxf(v, 0.0f);
      v += res[r];
      ((f16*)Y)[(int64_t)(rl + r) * N + col] = (f16)v;
    }
  } else {
    float* const y = (float*)Y + (OUT == kOutPartial ? (int64_t)split * M * N : 0);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (rl + r < M) y[(int64_t)(rl + r) * N + col] = a[r];
  }
}

// s_waitcnt that waits for at most n outstanding vector-memory operations (gfx9
// encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
#define DEC_WAIT_VM(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | ((((n) >> 4) & 3) << 14))
// Work-group barrier without a fence (a fence would wait for every load in flight).
// The bare barrier has no memory semantics for the compiler, so empty asm statements
// with a memory clobber keep LDS accesses from moving across it.
#define DEC_BARRIER()                  \
  do {                                 \
    asm volatile("" ::: "memory");     \
    __builtin_amdgcn_s_barrier();      \
    asm volatile("" ::: "memory");     \
  } while (0)

template <int MT16, int OUT>
__global__ __launch_bounds__(512, 1) void gemm_w4_dec_kernel(
    const f16* __restrict__ X, const uint8_t* __restrict__ Wc, const uint32_t* __restrict__ Wp,
    int M, int N, int K, int kt_per_split, int ntiles, Epilogue ep, void* __restrict__ Y) {
  using S = DecShape<MT16>;
  constexpr int NST = S::NST;
  __shared__ __attribute__((aligned(16))) uint8_t st0[S::STAGE_BYTES], st1[S::STAGE_BYTES],
      st2[S::STAGE_BYTES], st3[S::STAGE_BYTES], st4[S::STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;

  // work item: split-major, and each XCD (work-groups are dealt to the 8 XCDs in turn)
  // takes a contiguous range, so the work-groups sharing an L2 mostly share a k-range
  // of the activations
  const int total = ntiles * (int)gridDim.y;
  const int bid = blockIdx.x + blockIdx.y * gridDim.x;
  const int w = (total & 7) ? bid : (bid & 7) * (total >> 3) + (bid >> 3);
  const int split = w / ntiles;
  const int n0 = (w - split * ntiles) * S::BN;
  const int KT = K / kBK;
  const int kt0 = split * kt_per_split;
  const int kt1 = min(KT, kt0 + kt_per_split);

  // Buffer resources: X rows [0, M) and this block's three 128-row weight blocks (those
  // that exist: rows are allocated in whole blocks).  Row and block offsets in the
  // per-lane offset, the k-tile advance in the scalar offset: anything past the end is
  // out of range and reads zeros.  (The host keeps the byte counts below 2^31.)
  const int nblk = min((N - n0 + kW4BlockRows - 1) / kW4BlockRows, S::BN / kW4BlockRows);
  const rsrc_t x_rs = make_rsrc(X, M * K * 2);
  const rsrc_t w_rs = make_rsrc(Wc + w4_code_off(n0, 0, KT), nblk * KT * kW4TileBytes);
  const rsrc_t p_rs = make_rsrc(Wp + w4_param_idx(n0, 0, KT), nblk * KT * kW4BlockRows * 4);

  // Sixteen-byte slot i of this wave is instruction q = 4 wave + i of the stage: A rows
  // 8 q .. 8 q + 7, else codes rows 32 q' .. 32 q' + 31 (1 KB of one weight block's
  // contiguous 4 KB k-tile); the 4-byte slot of wave w < 6 loads params rows 64 w ..
  // 64 w + 63 (256 contiguous bytes).  A slot with nothing left repeats instruction
  // 0 of its kind (the same bytes to the same place), so every wave issues the same
  // loads and every target stays inside its stage.  All choices are wave-uniform.
#define DMA_SETUP(i)                                                                          \
  int q##i = 4 * wave + (i);                                                                  \
  if (q##i >= S::A_INSTR + S::C_INSTR) q##i = 0;                                              \
  const bool isa##i = q##i < S::A_INSTR;                                                      \
  const int qc##i = q##i - S::A_INSTR;                                                        \
  const int ar##i = 8 * q##i + (lane >> 3);                                                   \
  const rsrc_t rs##i = isa##i ? x_rs : w_rs;                                                  \
  const int km##i = isa##i ? 128 : kW4TileBytes;                                              \
  const int lo##i = isa##i ? q##i * 1024 : S::A_BYTES + qc##i * 1024;                         \
  const int vo##i = isa##i ? (ar##i * K + (((lane & 7) ^ ((ar##i >> 1) & 7)) << 3)) * 2       \
                           : (qc##i >> 2) * KT * kW4TileBytes + (qc##i & 3) * 1024 + lane * 16;
  DMA_SETUP(0) DMA_SETUP(1) DMA_SETUP(2) DMA_SETUP(3)
#undef DMA_SETUP
  const int qp = wave < S::P_INSTR ? wave : 0;
  const int lo4 = S::A_BYTES + S::C_BYTES + qp * 256;
  const int vo4 = ((qp >> 1) * KT * kW4BlockRows + (qp & 1) * 64 + lane) * 4;
#define LDSP(p) ((__attribute__((address_space(3))) void*)(p))
#define ISSUE(ST, KT)                                                                         \
  do {                                                                                        \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs0, LDSP(ST + lo0), 16, vo0, (KT) * km0, 0, 0); \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs1, LDSP(ST + lo1), 16, vo1, (KT) * km1, 0, 0); \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs2, LDSP(ST + lo2), 16, vo2, (KT) * km2, 0, 0); \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs3, LDSP(ST + lo3), 16, vo3, (KT) * km3, 0, 0); \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(p_rs, LDSP(ST + lo4), 4, vo4, (KT) * 512, 0, 0); \
  } while (0)

  f16x8 fbc[3], fbn[3];   // B fragments: this / next k-step
  constexpr bool kPf2 = MT16 % 3 == 0;
  f16x8 af[3];            // A fragments two row tiles ahead (kPf2)
  uint32_t cw0, cw1, cw2, pw0, pw1, pw2, t0, t1;
  f16x2 sp[3], mp[3];   // (scale, scale) and (offset, offset) of the 3 columns' group
  f32x4 acc[MT16][3];
#pragma unroll
  for (int i = 0; i < MT16; ++i)
#pragma unroll
    for (int t = 0; t < 3; ++t) acc[i][t] = (f32x4){0, 0, 0, 0};

  const int fa_base = ((lane & 15) * 64) * 2;                 // bytes
  const int f_sw = ((lane & 15) >> 1) & 7;
  const int c_off = S::A_BYTES + (48 * wave + (lane & 15)) * 32 + 4 * g;
  const int p_off = S::A_BYTES + S::C_BYTES + (48 * wave + (lane & 15)) * 4;

#define SB() __builtin_amdgcn_sched_barrier(0)
#define FRAG_A(ST, KS, i) \
  (*(const f16x8*)((ST) + fa_base + (i) * 16 * 128 + ((((4 * (KS) + g) ^ f_sw)) << 4)))
// code word WORD (0: k-step 0, 1: k-step 1) and params of the 3 column tiles
#define READ_W(ST, WORD)                                          \
  do {                                                            \
    cw0 = *(const uint32_t*)((ST) + c_off + 16 * (WORD));         \
    cw1 = *(const uint32_t*)((ST) + c_off + 512 + 16 * (WORD));   \
    cw2 = *(const uint32_t*)((ST) + c_off + 1024 + 16 * (WORD));  \
    if ((WORD) == 0) {                                            \
      pw0 = *(const uint32_t*)((ST) + p_off);                     \
      pw1 = *(const uint32_t*)((ST) + p_off + 64);                \
      pw2 = *(const uint32_t*)((ST) + p_off + 128);               \
    }                                                             \
  } while (0)
// word 0 of a k-tile (one 64-element group) expands the group's scale and offset into
// fp16 pairs; word 1 reuses them
#define DEQ(F, t, CW, PW, WORD)                                                     \
  do {                                                                              \
    if ((WORD) == 0) {                                                              \
      sp[t] = h2_from_u32(((PW) >> 16) * 0x10001u);                                 \
      mp[t] = h2_from_u32(((PW) & 0xFFFFu) * 0x10001u);                             \
    }                                                                               \
    w4_word_to_bytes(CW, t0, t1);                                                   \
    const f16x2 _d0 = dequant_pair(code_pair_f16<false>(t0), sp[t], mp[t]);         \
    const f16x2 _d1 = dequant_pair(code_pair_f16<true>(t0), sp[t], mp[t]);          \
    const f16x2 _d2 = dequant_pair(code_pair_f16<false>(t1), sp[t], mp[t]);         \
    const f16x2 _d3 = dequant_pair(code_pair_f16<true>(t1), sp[t], mp[t]);          \
    F[t] = (f16x8){_d0[0], _d0[1], _d1[0], _d1[1], _d2[0], _d2[1], _d3[0], _d3[1]}; \
  } while (0)
// one k-step: MT16 x 3 MFMAs with B fragments FB; after the MFMAs of row tile i: i = 0
// reads code words WORD of stage WST, i = 1..3 dequantize them into FN.  A fragments:
// when MT16 is a multiple of 3, row tile r of every k-step sits in af[r % 3], read two
// row tiles ahead, and the first two row tiles of the next k-step (k-step WORD of
// stage WST: this stage's k-step 1, or the next stage's k-step 0, whose loads the wait
// at the top of the k-tile has covered) are read during the last two row tiles of
// this one, so no k-step starts by waiting for LDS; otherwise one row tile ahead.
#define KSTEP(ST, KS, FB, FN, WST, WORD)                                                      \
  do {                                                                                        \
    if constexpr (kPf2) {                                                                     \
      _Pragma("unroll") for (int _i = 0; _i < MT16; ++_i) {                                  \
        if (_i + 2 < MT16) af[(_i + 2) % 3] = FRAG_A(ST, KS, _i + 2);                         \
        else af[(_i + 2) % 3] = FRAG_A(WST, WORD, _i + 2 - MT16);                             \
        const f16x8 _a = af[_i % 3];                                                          \
        acc[_i][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(_a, FB[0], acc[_i][0], 0, 0, 0); \
        acc[_i][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(_a, FB[1], acc[_i][1], 0, 0, 0); \
        acc[_i][2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(_a, FB[2], acc[_i][2], 0, 0, 0); \
        SB();                                                                                 \
        if (_i == 0) READ_W(WST, WORD);                                                       \
        if (_i == 1) DEQ(FN, 0, cw0, pw0, WORD);                                              \
        if (_i == 2) DEQ(FN, 1, cw1, pw1, WORD);                                              \
        if (_i == 3) DEQ(FN, 2, cw2, pw2, WORD);                                              \
        SB();                                                                                 \
      }                                                                                       \
    } else {                                                                                  \
      f16x8 _a0 = FRAG_A(ST, KS, 0), _a1 = _a0;                                               \
      _Pragma("unroll") for (int _i = 0; _i < MT16; ++_i) {                                  \
        if (_i + 1 < MT16) {                                                                  \
          if (_i & 1) _a0 = FRAG_A(ST, KS, _i + 1);                                           \
          else _a1 = FRAG_A(ST, KS, _i + 1);                                                  \
        }                                                                                     \
        const f16x8 _a = (_i & 1) ? _a1 : _a0;                                                \
        acc[_i][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(_a, FB[0], acc[_i][0], 0, 0, 0); \
        acc[_i][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(_a, FB[1], acc[_i][1], 0, 0, 0); \
        acc[_i][2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(_a, FB[2], acc[_i][2], 0, 0, 0); \
        SB();                                                                                 \
        if (_i == 0) READ_W(WST, WORD);                                                       \
        if (_i == 1) DEQ(FN, 0, cw0, pw0, WORD);                                              \
        if (_i == 2) DEQ(FN, 1, cw1, pw1, WORD);                                              \
        if (_i == 3) DEQ(FN, 2, cw2, pw2, WORD);                                              \
        SB();                                                                                 \
      }                                                                                       \
    }                                                                                         \
  } while (0)
// k-tile kt on stage ST (NXT: the stage of kt + 1, FREE: the stage of kt - 1, which
// receives kt + 4): wait until this wave's loads of kt + 1 have landed (all but the two
// later stages' 5 each), barrier, issue kt + 4, compute.  Past the last k-tile the
// issue repeats the last one (L2 hits; that stage is never read), so every k-tile
// issues exactly 5 loads and the counts stay exact.
#define TILE(ST, NXT, FREE)                                                                   \
  do {                                                                                        \
    DEC_WAIT_VM(S::SLOTS * (NST - 3));                                                        \
    DEC_BARRIER();                                                                            \
    ISSUE(FREE, min(kt + NST - 1, klast));                                                    \
    KSTEP(ST, 0, fbc, fbn, ST, 1);                                                            \
    KSTEP(ST, 1, fbn, fbc, NXT, 0);                                                           \
    ++kt;                                                                                     \
  } while (0)

  if (kt0 < kt1) {
    const int klast = kt1 - 1;
    int kt = kt0;
    ISSUE(st0, kt0);
    ISSUE(st1, min(kt0 + 1, klast));
    ISSUE(st2, min(kt0 + 2, klast));
    ISSUE(st3, min(kt0 + 3, klast));
    DEC_WAIT_VM(S::SLOTS * (NST - 2));
    DEC_BARRIER();
    READ_W(st0, 0);
    DEQ(fbc, 0, cw0, pw0, 0);
    DEQ(fbc, 1, cw1, pw1, 0);
    DEQ(fbc, 2, cw2, pw2, 0);
    if constexpr (kPf2) {
      af[0] = FRAG_A(st0, 0, 0);
      af[1] = FRAG_A(st0, 0, 1);
    }
    // whole groups of NST k-tiles, then the 0..NST-1 left over (starting on stage 0);
    // (a break after every k-tile makes the compiler spill the accumulators)
    for (; kt + NST - 1 <= klast;) {
      TILE(st0, st1, st4);
      TILE(st1, st2, st0);
      TILE(st2, st3, st1);
      TILE(st3, st4, st2);
      TILE(st4, st0, st3);
    }
    if (kt <= klast) TILE(st0, st1, st4);
    if (kt <= klast) TILE(st1, st2, st0);
    if (kt <= klast) TILE(st2, st3, st1);
    if (kt <= klast) TILE(st3, st4, st2);
    DEC_WAIT_VM(0);   // no load may land in LDS after the work-group ends
  }
#undef LDSP
#undef ISSUE
#undef SB
#undef FRAG_A
#undef READ_W
#undef DEQ
#undef KSTEP
#undef TILE

#pragma unroll
  for (int i = 0; i < MT16; ++i)
#pragma unroll
    for (int t = 0; t < 3; ++t)
      store_acc16<OUT>(acc[i][t], i * 16, n0 + 48 * wave + 16 * t + (lane & 15), M, N, ep, Y,
                       split);
}
#undef DEC_WAIT_VM
#undef DEC_BARRIER

// Sum of split-K partials in split order, then the epilogue.  4 elements per thread.
template <int OUT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int splits, int M, int N, Epilogue ep,
                                                            void* __restrict__ Y) {
  const int64_t total = (int64_t)M * N;
  const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i4 >= total) return;
  float v[4] = {0, 0, 0, 0};
  for (int z = 0; z < splits; ++z) {
    const float4 p = *(const float4*)(part + (int64_t)z * total + i4);
    v[0] += p.x;
    v[1] += p.y;
    v[2] += p.z;
    v[3] += p.w;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t idx = i4 + e;
    const int64_t row = idx / N;
    const int col = (int)(idx - row * N);
    if constexpr (OUT == kOutF16)
      ((f16*)Y)[idx] = (f16)epilogue_value(v[e], ep, row, col, N);
    else
      ((float*)Y)[idx] = v[e];
  }
}

// ------------------------------------------------------------------ host dispatch

}  // namespace flexq

#include "host_cache.h"

namespace flexq {

struct Plan {
  int cfg;      // which kernel / tile shape
  int bm, bn;
  int splits;
  int kt_per_split;
};

constexpr int kCfgBig = 0;      // M > 160: 256 x 256 tile, 8 waves (pipelined, dequant into LDS)
constexpr int kCfgSkinny = 1;   // M <= 64 or 144 < M <= 160: 32*ceil(M/32) x 256 tile
constexpr int kCfgDec = 2;      // 64 < M <= 144: 16*ceil(M/16) x 384 tile, 8 waves

// Work-groups of the small-M kernels that one device runs at once (occupancy x CUs),
// looked up once per device and tile height.
template <int MT>
static int skinny_blocks_per_cu() {
  static PerDeviceInt cache;
  return cache.get([] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &b, gemm_w4_skinny_kernel<MT, 4, 2, kOutPartial>, 256,
            SkinnyShape<MT, 4, 2>::LDS_BYTES) != hipSuccess)
      return 0;
    return b;
  }, 1);
}

template <int MT16>
static int dec_blocks_per_cu() {
  static PerDeviceInt cache;
  return cache.get([] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, gemm_w4_dec_kernel<MT16, kOutPartial>,
                                                     512, 0) != hipSuccess)
      return 0;
    return b;
  }, 1);
}

static int device_cus() {
  static PerDeviceInt cache;
  return cache.get([] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    return n;
  }, 256);
}

static int64_t dec_concurrency(int mt16) {
  int per_cu = 1;
  switch (mt16) {
    case 5: per_cu = dec_blocks_per_cu<5>(); break;
    case 6: per_cu = dec_blocks_per_cu<6>(); break;
    case 7: per_cu = dec_blocks_per_cu<7>(); break;
    case 8: per_cu = dec_blocks_per_cu<8>(); break;
    default: per_cu = dec_blocks_per_cu<9>(); break;
  }
  return (int64_t)per_cu * device_cus();
}

static int64_t skinny_concurrency(int mt) {
  int per_cu = 1;
  switch (mt) {
    case 1: per_cu = skinny_blocks_per_cu<1>(); break;
    case 2: per_cu = skinny_blocks_per_cu<2>(); break;
    case 3: per_cu = skinny_blocks_per_cu<3>(); break;
    case 4: per_cu = skinny_blocks_per_cu<4>(); break;
    default: per_cu = skinny_blocks_per_cu<5>(); break;
  }
  return (int64_t)per_cu * device_cus();
}

static Plan make_plan(int64_t M, int64_t N, int64_t K, size_t ws_bytes) {
  Plan p;
  // (the decode kernel addresses X and its 384 W rows with 32-bit buffer offsets)
  if (M > 64 && M <= 144 && K <= (1 << 22)) { p.cfg = kCfgDec; p.bm = (int)((M + 15) / 16) * 16; p.bn = 384; }
  else if (M <= 160) { p.cfg = kCfgSkinny; p.bm = (int)((M + 31) / 32) * 32; p.bn = 256; }
  else { p.cfg = kCfgBig; p.bm = 256; p.bn = 256; }
  const int64_t KT = K / kBK;
  const int64_t tiles = ((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
  int splits = 1;
  if (p.cfg == kCfgSkinny || p.cfg == kCfgDec) {
    // Split-K count of the small-M kernels from a cost model fitted on MI355X at the
    // decode shapes: time ~ rounds of resident work-groups x (a fixed cost of ~16
    // k-tiles per work-group + its k-tiles) + the partial sums written and reduced
    // (~4.75 MB per k-tile time).  Rounds matter: 576 work-groups on 256 CUs cost as
    // much as 768.
    const int64_t conc = p.cfg == kCfgDec ? dec_concurrency(p.bm / 16) : skinny_concurrency(p.bm / 32);
    double best = 1e300;
    for (int64_t s = 1; s <= 8 && s <= KT; ++s) {
      const int64_t kps = (KT + s - 1) / s;
      const int64_t sp = (KT + kps - 1) / kps;
      const int64_t rounds = (tiles * sp + conc - 1) / conc;
      double c = (double)rounds * (double)(16 + kps);
      if (sp > 1) c += (double)sp * (double)M * (double)N * 4.0 / 4.75e6;
      if (c < best) {
        best = c;
        splits = (int)sp;
      }
    }
  } else if (tiles < 512) {
    // too few work-groups for 256 CUs: split K (a fixed rule, so results depend only
    // on the shape and on whether the workspace is large enough)
    splits = (int)((512 + tiles - 1) / tiles);
    splits = (int)std::min<int64_t>(splits, std::max<int64_t>(1, KT / 8));
    splits = std::min(splits, 16);
  }
  if ((M * N) % 4) splits = 1;
  while (splits > 1 && (size_t)splits * M * N * sizeof(float) > ws_bytes) --splits;
  p.splits = splits;
  p.kt_per_split = (int)((KT + splits - 1) / splits);
  p.splits = (int)((KT + p.kt_per_split - 1) / p.kt_per_split);
  return p;
}

template <int WM, int WN, int TM, int TN, int OUT>
static void launch_big(const Plan& p, const f16* x, const flexq_w4* W, int M, Epilogue ep,
                       void* Y, hipStream_t stream) {
  using S = GemmShape<WM, WN, TM, TN>;
  auto kern = gemm_w4_big_kernel<WM, WN, TM, TN, OUT>;
  static PerDeviceInt attr_set;   // the dynamic LDS limit, raised once per device
  (void)attr_set.get([&] {
    return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)S::LDS_BYTES) == hipSuccess ? 1 : 0;
  }, 0);
  const int N = (int)W->rows, K = (int)W->cols;
  const int tiles = ((M + S::BM - 1) / S::BM) * ((N + S::BN - 1) / S::BN);
  dim3 grid(tiles, p.splits);
  hipLaunchKernelGGL(kern, grid, dim3(S::THREADS), S::LDS_BYTES, stream, x, W->codes,
                     (const uint32_t*)W->params, M, N, K, p.kt_per_split, ep, Y);
}

template <int MT16, int OUT>
static void launch_dec(const Plan& p, const f16* x, const flexq_w4* W, int M, Epilogue ep,
                       void* Y, hipStream_t stream) {
  using S = DecShape<MT16>;
  const int N = (int)W->rows, K = (int)W->cols;
  const int ntiles = (N + S::BN - 1) / S::BN;
  dim3 grid(ntiles, p.splits);
  hipLaunchKernelGGL((gemm_w4_dec_kernel<MT16, OUT>), grid, dim3(S::THREADS), 0, stream, x,
                     W->codes, (const uint32_t*)W->params, M, N, K, p.kt_per_split, ntiles, ep, Y);
}

template <int MT, int OUT>
static void launch_skinny(const Plan& p, const f16* x, const flexq_w4* W, int M, Epilogue ep,
                          void* Y, hipStream_t stream) {
  constexpr int NW = 4, TN = 2;
  using S = SkinnyShape<MT, NW, TN>;
  auto kern = gemm_w4_skinny_kernel<MT, NW, TN, OUT>;
  const int N = (int)W->rows, K = (int)W->cols;
  dim3 grid((N + S::BN - 1) / S::BN, p.splits, (M + S::BM - 1) / S::BM);
  hipLaunchKernelGGL(kern, grid, dim3(S::THREADS), S::LDS_BYTES, stream, x, W->codes,
                     (const uint32_t*)W->params, M, N, K, p.kt_per_split, ep, Y);
}

template <int OUT>
static void launch_plan(const Plan& p, const f16* x, const flexq_w4* W, int M, Epilogue ep,
                        void* Y, hipStream_t stream) {
  if (p.cfg == kCfgDec) {
    switch (p.bm / 16) {
      case 5: launch_dec<5, OUT>(p, x, W, M, ep, Y, stream); break;
      case 6: launch_dec<6, OUT>(p, x, W, M, ep, Y, stream); break;
      case 7: launch_dec<7, OUT>(p, x, W, M, ep, Y, stream); break;
      case 8: launch_dec<8, OUT>(p, x, W, M, ep, Y, stream); break;
      default: launch_dec<9, OUT>(p, x, W, M, ep, Y, stream); break;
    }
  } else if (p.cfg == kCfgSkinny) {
    switch (p.bm / 32) {
      case 1: launch_skinny<1, OUT>(p, x, W, M, ep, Y, stream); break;
      case 2: launch_skinny<2, OUT>(p, x, W, M, ep, Y, stream); break;
      case 3: launch_skinny<3, OUT>(p, x, W, M, ep, Y, stream); break;
      case 4: launch_skinny<4, OUT>(p, x, W, M, ep, Y, stream); break;
      default: launch_skinny<5, OUT>(p, x, W, M, ep, Y, stream); break;
    }
  } else {
    launch_big<2, 4, 4, 2, OUT>(p, x, W, M, ep, Y, stream);
  }
}

static int check_w4(const flexq_w4* W) {
  if (!W || !W->codes || !W->params) return FLEXQ_ERR_INVALID;
  if (W->rows <= 0 || W->cols <= 0 || W->cols % kBK) return FLEXQ_ERR_INVALID;
  if (W->rows > 0x7FFFFFFF || W->cols > 0x7FFFFFFF) return FLEXQ_ERR_UNSUPPORTED;
  if (((uintptr_t)W->codes & 15) || ((uintptr_t)W->params & 3)) return FLEXQ_ERR_INVALID;
  return FLEXQ_OK;
}

static int run_linear(const uint16_t* x, int64_t M, const flexq_w4* W, Epilogue ep, int out_kind,
                      void* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_w4(W);
  if (st != FLEXQ_OK) return st;
  if (M < 0 || M > 0x7FFFFFFF) return FLEXQ_ERR_INVALID;
  if (M == 0) return FLEXQ_OK;
  if (!x || !y || ((uintptr_t)x & 15)) return FLEXQ_ERR_INVALID;
  const Plan p = make_plan(M, W->rows, W->cols, ws ? ws_bytes : 0);
  const f16* xh = (const f16*)x;
  if (p.splits == 1) {
    if (out_kind == kOutF16) launch_plan<kOutF16>(p, xh, W, (int)M, ep, y, stream);
    else launch_plan<kOutF32>(p, xh, W, (int)M, ep, y, stream);
  } else {
    const int64_t total = M * W->rows;
    if (((uintptr_t)ws & 15) || total % 4) return FLEXQ_ERR_INVALID;
    launch_plan<kOutPartial>(p, xh, W, (int)M, ep, ws, stream);
    const int64_t blocks = (total / 4 + 255) / 256;
    if (out_kind == kOutF16)
      hipLaunchKernelGGL(splitk_reduce_kernel<kOutF16>, dim3((unsigned)blocks), dim3(256), 0, stream,
                         (const float*)ws, p.splits, (int)M, (int)W->rows, ep, y);
    else
      hipLaunchKernelGGL(splitk_reduce_kernel<kOutF32>, dim3((unsigned)blocks), dim3(256), 0, stream,
                         (const float*)ws, p.splits, (int)M, (int)W->rows, ep, y);
  }
  FLEXQ_LAUNCH_CHECK();
  return FLEXQ_OK;
}

}  // namespace flexq

using namespace flexq;

extern "C" size_t flexq_linear_w4_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % kBK) return 0;
  const Plan p = make_plan(M, N, K, (size_t)-1);
  return p.splits > 1 ? (size_t)p.splits * M * N * sizeof(float) : 0;
}

extern "C" int flexq_linear_w4(const uint16_t* x, int64_t M, const flexq_w4* W, const uint16_t* bias,
                               const uint16_t* residual, int32_t relu, uint16_t* y, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  Epilogue ep{(const f16*)bias, (const f16*)residual, relu ? 1 : 0};
  return run_linear(x, M, W, ep, kOutF16, y, ws, ws_bytes, stream);
}

extern "C" int flexq_linear_w4_f32(const uint16_t* x, int64_t M, const flexq_w4* W, float* y32,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  Epilogue ep{nullptr, nullptr, 0};
  return run_linear(x, M, W, ep, kOutF32, y32, ws, ws_bytes, stream);
}
