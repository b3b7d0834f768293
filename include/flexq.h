/*
 * flexq — group-wise 4-bit weight + KV-cache OPT decoder path on MI355X (gfx950).
 *
 * C ABI of the HIP library libflexq.so.
 *
 * Conventions shared by every call
 *   - fp16 values travel as uint16_t bit patterns (IEEE binary16).
 *   - Every pointer argument is a DEVICE pointer owned by the caller, unless the
 *     comment says "host".  The library never allocates, frees or keeps device
 *     memory; scratch space comes in through an explicit workspace argument whose
 *     required size a *_workspace_size() call reports.
 *   - Arrays are row-major, innermost dimension contiguous.
 *   - Calls check their arguments on the host, then enqueue their kernels on
 *     `stream` and return without waiting.  A rejected call enqueues nothing.
 *     A launch failure reported by the runtime returns FLEXQ_ERR_DEVICE; a fault
 *     inside a kernel surfaces at the caller's next synchronisation.
 *   - No state is kept between calls except host-side, per-device caches of launch
 *     facts (occupancy, CU count, raised LDS limits), looked up once per device and
 *     published atomically.  Calls on distinct streams and buffers may run
 *     concurrently, from any thread.
 *   - Results are deterministic: fixed reduction and merge orders, chosen from the
 *     shapes, the workspace size and the device's CU count and occupancy only.
 *
 * Compressed formats (FlexGen source walkthrough, section 6.3: num_bits 4,
 * group_size 64, asymmetric; weights grouped along group_dim 0, the cache along
 * group_dim 2; codes packed two per byte next to one fp16 parameter tensor)
 *   - A group is 64 consecutive elements of the innermost dimension.
 *   - codes:  uint8 [..][cols/2]; element 2j in the low nibble of byte j,
 *             element 2j+1 in the high nibble.
 *   - params: uint16 [..][cols/64][2] = (offset, scale) as fp16 per group; the
 *             value of code c is c * scale + offset (scale = (max - min) / 15,
 *             offset = min).  0.5625 bytes per element in total.
 */
#ifndef FLEXQ_H
#define FLEXQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FLEXQ_OK = 0,
  FLEXQ_ERR_INVALID = -1,     /* bad pointer, size, layout or workspace too small */
  FLEXQ_ERR_UNSUPPORTED = -2, /* a valid configuration this build does not implement */
  FLEXQ_ERR_DEVICE = -3       /* the HIP runtime reported an error at launch */
} flexq_status;

/* CompressionConfig of the pages (walkthrough section 6.3).  This build accepts
 * {num_bits 4, group_size 64, symmetric 0} and returns FLEXQ_ERR_UNSUPPORTED for
 * anything else. */
typedef struct {
  int32_t num_bits;
  int32_t group_size;
  int32_t symmetric;
} flexq_qconfig;

/* A 4-bit weight matrix W[rows][cols] (rows = N outputs, cols = K inputs), grouped
 * along cols (one group = 64 columns = one k-tile), in the weight layout written by
 * flexq_quantize_w4: rows in blocks of FLEXQ_W4_BLOCK_ROWS = 128, and within block b
 * the k-tiles in order, each holding the block's 128 rows contiguously:
 *   codes  byte  ((r / 128) * (cols/64) + kt) * 4096 + (r % 128) * 32 + 4 q + j
 *          holds elements 64 kt + 8 q + j (low nibble) and 64 kt + 8 q + j + 4 (high
 *          nibble) of row r (q = 0..7, j = 0..3: within each 32-bit word the
 *          low nibbles hold its first four codes, so spreading a word to one code per
 *          byte takes one AND and one shift);
 *   params word  ((r / 128) * (cols/64) + kt) * 128 + (r % 128) = (offset, scale)
 *          as two fp16 (offset in the low half) of group kt of row r.
 * Both arrays cover rows padded up to a multiple of 128 (FLEXQ_W4_CODES_BYTES /
 * FLEXQ_W4_PARAMS_BYTES); pad rows hold zeros.  Codes and params are those of
 * flexq_quantize, only their order differs: a k-tile of any run of rows is read in
 * whole cache lines, which streaming the weights at small batch needs, and a code
 * word expands to fp16 with two fewer instructions. */
#define FLEXQ_W4_BLOCK_ROWS 128
#define FLEXQ_W4_CODES_BYTES(rows, cols) \
  ((((rows) + 127) / 128) * 128 * (int64_t)(cols) / 2)
#define FLEXQ_W4_PARAMS_BYTES(rows, cols) \
  ((((rows) + 127) / 128) * 128 * (int64_t)(cols) / 16)
typedef struct {
  const uint8_t* codes;
  const uint16_t* params;
  int64_t rows;
  int64_t cols;
} flexq_w4;

/* The 4-bit KV cache of one layer.  Groups are 64 consecutive head_dim elements
 * of one token's K (or V) vector in one head.
 *   k_codes, v_codes   [batch][heads][max_len][head_dim/2]
 *   k_params, v_params [batch][heads][max_len][head_dim/64][2]
 *   pad                NULL, or device int32 [batch]: left padding of each cache row
 *                      (ragged prompts; source notes "Flex Opt", the attention mask of
 *                      generate).  Positions [0, pad) of the row hold pad tokens:
 *                      attention never reads them, and a pad query's prefill output is
 *                      0.  Valid values lie in [0, prompt length); others are clamped
 *                      to [0, S - 1] at prefill and [0, pos] at decode.  Read by the
 *                      kernels when they run, so it may change between calls. */
typedef struct {
  uint8_t* k_codes;
  uint8_t* v_codes;
  uint16_t* k_params;
  uint16_t* v_params;
  int32_t batch;
  int32_t heads;
  int32_t head_dim; /* 64 or 128 */
  int32_t max_len;
  const int32_t* pad;
} flexq_kv4_layer;

/* Weights of one pre-LayerNorm OPT decoder layer (source notes, "Flex Opt": the
 * model is an embedding, N transformer layers and an output head).  fp16 vectors
 * of length hidden (LN gains/biases, bo, b2), 3*hidden (bqkv) or ffn (b1).
 * wqkv [3h][h] produces [Q | K | V], each head-major (head * head_dim + d). */
typedef struct {
  const uint16_t *ln1_g, *ln1_b;
  flexq_w4 wqkv;
  const uint16_t* bqkv;
  flexq_w4 wo;
  const uint16_t* bo;
  const uint16_t *ln2_g, *ln2_b;
  flexq_w4 w1;
  const uint16_t* b1;
  flexq_w4 w2;
  const uint16_t* b2;
} flexq_layer;

/* Optional launch timing: when a model carries a trace, flexq_prefill and
 * flexq_decode_step record events[2i] / events[2i+1] on their stream right before
 * and after each 4-bit linear layer they launch (split-K reduction included) and
 * note which one in kinds[i] (FLEXQ_TRACE_*) and its row count in rows[i].  The
 * caller creates the 2*capacity events (HOST array) and resets count; recording
 * stops silently when count reaches capacity. */
enum { FLEXQ_TRACE_QKV = 0, FLEXQ_TRACE_OUT = 1, FLEXQ_TRACE_FC1 = 2, FLEXQ_TRACE_FC2 = 3,
       FLEXQ_TRACE_HEAD = 4 };
typedef struct {
  hipEvent_t* events;
  int32_t* kinds;
  int64_t* rows;
  int32_t capacity;
  int32_t count;
} flexq_trace;

/* Token choice of a generation (walkthrough section 4.1, `generate(..., do_sample,
 * temperature, ..., stop)`; source notes "Flex Opt": the Task's temperature and
 * stop token, the per-sequence stopped flags).
 *   do_sample 0: greedy, the largest logit (lowest index among equal maxima).
 *   do_sample 1: a draw from softmax(logits / temperature) by the Gumbel-max rule:
 *     argmax_n (logit_n / T - log(-log u_n)) in fp64, lowest index on ties, with
 *     u_n = ((z >> 12) + 1/2) 2^-52 and z the SplitMix64 output number
 *     step * 2^48 + sequence * 2^32 + n from state `seed` (seed + (c + 1) *
 *     0x9E3779B97F4A7C15, then the published mix).  The draw depends only on
 *     (seed, step, sequence, n): not on the batch split or the launch.
 *   stop: a token id in [0, vocab), or -1 for none.  A sequence that emits it is
 *     stopped and emits it at every later step. */
typedef struct {
  int32_t do_sample;
  float temperature; /* > 0 and finite when do_sample */
  uint64_t seed;
  int32_t stop;
} flexq_gen_config;

/* Host-DRAM tier of the KV cache (source notes "Flex Opt": cache placement between
 * GPU and CPU, the cpu_cache_compute policy, and the load_cache path that splits a
 * batch's attention between the GPU and the CPU).  Model cache rows >= row0 live in
 * HOST memory (host row r - row0), for batches whose 4-bit cache does not fit in
 * HBM; rows < row0 stay in the device caches `kv`.  A decode step copies the host
 * rows' q, k, v to host_ws, runs their attention on the CPU (threads, as
 * flexq_host_attn_decode_kv4) while the GPU attends the device rows, and copies
 * the outputs back: the call blocks the host once per layer and cannot be captured
 * in a graph.  A prefill micro-batch must lie wholly on one side of row0; a host
 * micro-batch writes its K/V to the device `stage` area, then copies them to the
 * host caches.  With left padding, kv[0].pad must hold all model rows (the
 * embedding reads it) and each kv[l] of the host tier its own host rows' pads.
 *   kv        HOST array of `layers` caches in pinned HOST memory (batch = host rows)
 *   host_ws   pinned HOST memory, >= (decode batch - row0) * 4 * hidden * 2 bytes
 *   stage     DEVICE memory, >= flexq_host_stage_size(heads, head_dim, nb, max_len)
 *             for the largest host prefill micro-batch nb (max_len of the host tier) */
typedef struct {
  const flexq_kv4_layer* kv;
  int32_t row0;
  int32_t threads; /* CPU threads for the host rows' attention (<= 0: all) */
  void* host_ws;
  size_t host_ws_bytes;
  void* stage;
  size_t stage_bytes;
} flexq_host_tier;

size_t flexq_host_stage_size(int32_t heads, int32_t head_dim, int32_t nb, int32_t max_len);

/* Optional copies of the hidden states between layers, for checking a whole run
 * layer by layer (the engine's layer loop of source notes "Flex Opt" keeps each
 * layer's input and output in one hidden buffer; a tap copies that buffer out).
 * When a model carries a tap, flexq_prefill and flexq_decode_step copy, on their
 * stream, the input of layer layers[i] (all rows of the call, rows x hidden fp16)
 * into x[i]; layers[i] == the model's layer count names the last layer's output
 * (the input of the final LayerNorm).  A call with more rows than rows_cap, or a
 * layer index outside [0, layers], returns FLEXQ_ERR_INVALID before any work. */
typedef struct {
  int32_t count;
  const int32_t* layers; /* HOST [count] */
  uint16_t* const* x;    /* HOST [count] of DEVICE buffers, rows_cap * hidden fp16 each */
  int64_t rows_cap;
} flexq_tap;

/* A whole OPT-shaped model.  Non-owning: every pointer stays the caller's.
 * `layer` and `kv` are HOST arrays of `layers` entries (the structs inside hold
 * device pointers).  embed is the 4-bit token embedding [vocab][hidden], also used
 * as the LM head (tied, no bias).  pos is the fp16 learned-position table
 * [pos_rows][hidden]; position p reads row p + 2.  workspace must hold
 * flexq_model_workspace_size(...) bytes. */
typedef struct {
  int32_t layers, hidden, heads, ffn, vocab, pos_rows;
  const flexq_layer* layer;
  const flexq_kv4_layer* kv;
  flexq_w4 embed;
  const uint16_t* pos;
  const uint16_t *lnf_g, *lnf_b;
  void* workspace;
  size_t workspace_bytes;
  flexq_trace* trace; /* NULL, or a HOST trace (see flexq_trace) */
  /* NULL (greedy), or a HOST generation config; step = the position of the token
   * whose logits are drawn from (prompt length - 1 at prefill, pos at decode),
   * sequence = the cache row. */
  const flexq_gen_config* gen;
  /* NULL, or device int32 [cache batch]: stopped flag of each cache row, set by
   * flexq_prefill from the first token and kept by flexq_decode_step (needs a stop
   * token in gen). */
  int32_t* stopped;
  /* decode attention: dense unless 0 < attn_sparsity < 1, then top-k sparse (see
   * flexq_attn_decode_kv4_topk) */
  float attn_sparsity;
  /* NULL, or a HOST host-tier description (see flexq_host_tier); not combined with
   * sparse attention */
  const flexq_host_tier* host;
  /* NULL, or a HOST tap description (see flexq_tap) */
  const flexq_tap* tap;
} flexq_model;

const char* flexq_status_string(int status);

/* ---------------------------------------------------------------- quantize/pack
 * Group-wise min/max asymmetric 4-bit quantization (walkthrough section 6.3,
 * `compress`).  x fp16 [rows][cols], cols a multiple of 64, values finite.
 * Writes codes [rows][cols/2] and params [rows][cols/64][2].  Per group, in fp32:
 * step = fp16(fl32(max - min) / 15) (0 for a constant group, 2^-24 if the step
 * underflows), code = clamp(rne(fl32(x - min) * fl32(1 / step)), 0, 15), offset =
 * min with a zero stored as +0.  Bit-identical to the oracle on identical input. */
int flexq_quantize(const uint16_t* x, int64_t rows, int64_t cols, flexq_qconfig cfg,
                   uint8_t* codes, uint16_t* params, hipStream_t stream);

/* The same quantization as flexq_quantize, written in the 4-bit weight layout of
 * flexq_w4 (codes FLEXQ_W4_CODES_BYTES(rows, cols) bytes, params
 * FLEXQ_W4_PARAMS_BYTES(rows, cols) bytes, pad rows written as zeros).  codes 8-byte
 * and params 4-byte aligned; same errors as flexq_quantize. */
int flexq_quantize_w4(const uint16_t* x, int64_t rows, int64_t cols, flexq_qconfig cfg,
                      uint8_t* codes, uint16_t* params, hipStream_t stream);

/* General compression config (walkthrough section 6.3 names num_bits, group_size,
 * group_dim and symmetric; the hub page mentions int3/int4).  x fp16 seen as
 * [outer][n][inner], grouped along n in groups of cfg.group_size consecutive positions
 * (inner = 1 when the grouped axis is the innermost one; any other group_dim is the
 * product split of the shape around it).  cfg: num_bits 2..8, group_size 1..4096 with
 * group_size * num_bits a multiple of 8, symmetric 0 or 1; else FLEXQ_ERR_UNSUPPORTED.
 * A ragged last group is zero-padded and the padding quantized with it.  Per group,
 * fp32, contraction off:
 *   asymmetric: step = fp16((max - min) / (2^b - 1)), code = clamp(rne((x - min) *
 *               (1 / step)), 0, 2^b - 1), offset = min (+0 for a zero minimum);
 *   symmetric:  B = 2^(b-1) - 1, step = fp16(max|x| / B), code = clamp(rne(x * (1 /
 *               step)), -B, B) + 2^(b-1), offset = +0;
 *   constant (asymmetric) / all-zero (symmetric) group: step 0; a step that
 *   underflows fp16 becomes 2^-24.
 * Outputs (ng = ceil(n / group_size), gb = group_size * num_bits / 8):
 *   codes  uint8 [outer][ng * gb][inner]: the b-bit codes of a group concatenated
 *          least significant bit first into gb bytes along n;
 *   params (offset, step) fp16 pairs [outer][ng][inner].
 * x 2-byte and params 4-byte aligned; bit-identical to the oracle. */
int flexq_quantize_ex(const uint16_t* x, int64_t outer, int64_t n, int64_t inner,
                      flexq_qconfig cfg, uint8_t* codes, uint16_t* params, hipStream_t stream);

/* Inverse of flexq_quantize_ex: out fp16 [outer][n][inner] = fp16(code * step + offset),
 * or fp16((code - 2^(b-1)) * step) if symmetric, one rounding of the exact value; the
 * padding of a ragged last group is not written. */
int flexq_dequantize_ex(const uint8_t* codes, const uint16_t* params, int64_t outer, int64_t n,
                        int64_t inner, flexq_qconfig cfg, uint16_t* out, hipStream_t stream);

/* Inverse of flexq_quantize (row-major codes and params, `decompress`): out fp16 [rows][cols] =
 * fp16(code * scale + offset) with one rounding.  A test and inspection aid; the
 * GEMMs dequantize inside their own tiles. */
int flexq_dequantize(const uint8_t* codes, const uint16_t* params, int64_t rows, int64_t cols,
                     uint16_t* out, hipStream_t stream);

/* ---------------------------------------------------------------- LayerNorm
 * The layer norms of the OPT decoder stack (source notes, "Flex Opt": the model is an
 * embedding, N transformer layers and an output head; the pages name the layers but
 * not their norm, so this follows the OPT architecture: pre-LN twice per layer and a
 * final norm before the head).
 * y[m] = (x[m] - mean) / sqrt(biased var + 1e-5) * g + b, statistics in fp32,
 * fp16 out.  Row m of x starts at x + m * x_row_stride (elements); y is dense
 * [M][h].  h a multiple of 8 up to FLEXQ_LN_MAX_HIDDEN, the stride a multiple of 8
 * and >= h, x, g, b, y 16-byte aligned and not NULL, M >= 0 (M = 0 does nothing);
 * anything else -> FLEXQ_ERR_INVALID. */
#define FLEXQ_LN_MAX_HIDDEN 16384
int flexq_layernorm(const uint16_t* x, int64_t M, int64_t h, int64_t x_row_stride,
                    const uint16_t* g, const uint16_t* b, uint16_t* y, hipStream_t stream);

/* ---------------------------------------------------------------- 4-bit linear
 * A linear layer of the decoder with its weight compressed group-wise (walkthrough
 * section 6.3: weights compressed to 4 bits in groups of 64 along group_dim 0, the
 * input dimension, and decompressed to the original fp16 for the layer's matmul;
 * source notes "Pytorch Backend": a compressed weight is the (codes, scale, shape)
 * triple that the backend decompresses before use).  Here the decompression happens
 * inside the GEMM's tiles and the weight is never materialised:
 * y[M][N] = fp16( [relu](x . W^T + bias) [+ residual] ), W = the fp16 value
 * fp16(code * scale + offset) of every 4-bit weight [N][K] (one rounding).
 * x fp16 [M][K] (16-byte aligned); bias fp16 [N] or NULL; residual fp16 [M][N] or
 * NULL (may equal y); relu 0/1.  fp16 MFMA operands, fp32 accumulation, one rounding
 * at the end.  K a multiple of 64, else FLEXQ_ERR_INVALID.  ws: scratch for split-K
 * partial sums (16-byte aligned); flexq_linear_w4_workspace_size(M, N, K) bytes give
 * the fastest split; a smaller workspace (NULL and 0 included) is accepted and runs
 * with as many splits as fit (fewer or none): the same error bound, another (fixed)
 * summation order. */
size_t flexq_linear_w4_workspace_size(int64_t M, int64_t N, int64_t K);
int flexq_linear_w4(const uint16_t* x, int64_t M, const flexq_w4* W, const uint16_t* bias,
                    const uint16_t* residual, int32_t relu, uint16_t* y, void* ws,
                    size_t ws_bytes, hipStream_t stream);

/* Same product written as fp32 without bias, activation or rounding: y32 [M][N].
 * Used for logits against the tied embedding (`opt_output_embed`). */
int flexq_linear_w4_f32(const uint16_t* x, int64_t M, const flexq_w4* W, float* y32,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- attention
 * Prefill attention (source notes, "Pytorch Backend": `mha`).  qkv fp16
 * [B*S][3h], rows ordered (b, t).  For each sequence and head: causal
 * softmax(q k^T / sqrt(head_dim)) v over the fp16 K/V of this pass, output fp16
 * out [B*S][h].  Scores, their maximum and the softmax sums are fp32; the
 * probabilities multiply V as fp16 MFMA operands (each p in [0, 1] rounded once to
 * fp16, relative error <= 2^-11) with fp32 accumulation, so the output may differ
 * from an all-fp32 softmax by up to about 2^-11 max|v| beyond the final rounding.  K and V of the S positions are then
 * quantized into cache rows b0 .. b0+B-1, positions [0, S).  Needs
 * b0 + B <= kv->batch and S <= kv->max_len. */
int flexq_attn_prefill(const uint16_t* qkv, int32_t B, int32_t S, int32_t b0,
                       const flexq_kv4_layer* kv, uint16_t* out, hipStream_t stream);

/* Decode attention over the 4-bit cache (`mha_gen`).  qkv fp16 [B][3h], one new
 * token per sequence for cache rows b0 .. b0+B-1.  The token's k, v are quantized
 * into position pos, then positions [0, pos] are read back from the cache (codes
 * dequantized to fp32), softmax in fp32, output fp16 out [B][h].  The context is
 * split over work-groups (split-K) and merged with an online-softmax rescale in a
 * fixed order.  ws: at least flexq_attn_decode_workspace_size(...) bytes. */
size_t flexq_attn_decode_workspace_size(int32_t B, int32_t heads, int32_t head_dim, int32_t pos);
int flexq_attn_decode_kv4(const uint16_t* qkv, int32_t B, int32_t b0, int32_t pos,
                          const flexq_kv4_layer* kv, uint16_t* out, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* Decode attention that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same computation, kernels and result bits as flexq_attn_decode_kv4,
 * with the context-split partials in a static device array of
 * FLEXQ_STATIC_SCRATCH_BYTES that each device holds from the call's first use on it
 * until the process ends (its address is looked up once per device).  Needs
 * flexq_attn_decode_workspace_size(B, heads, head_dim, pos) <=
 * FLEXQ_STATIC_SCRATCH_BYTES (4 MiB; the size is 0 when B x heads >= 1024 and
 * pos < 4096, and at most about 1.1 MB when B x heads < 1024 and pos + 1 <=
 * 2^22 / (B x heads)), else FLEXQ_ERR_UNSUPPORTED before any work;
 * FLEXQ_ERR_DEVICE if the array's device address cannot be obtained.  Every call on
 * one device shares that device's array: calls that overlap in time on one device
 * (two streams, two threads) race on it and must be ordered by the caller.  Each
 * call writes every partial it reads, so nothing carries over from a previous call
 * and nothing needs clearing. */
#define FLEXQ_STATIC_SCRATCH_BYTES (4u << 20)
int flexq_attn_decode_kv4_static(const uint16_t* qkv, int32_t B, int32_t b0, int32_t pos,
                                 const flexq_kv4_layer* kv, uint16_t* out, hipStream_t stream);

/* Sparse decode attention (source notes "Flex Opt": the `attn_sparsity` policy, whose
 * mechanism the pages leave open).  As flexq_attn_decode_kv4, except that each query
 * keeps only the k = max(1, ceil(min(sparsity, 1) * n)) highest of its n scores
 * (n = pos + 1 - pad, the product in fp32; among equal scores the lower position
 * first) and takes the softmax over those alone.  One work-group per (sequence,
 * head), no workspace; needs pos + 1 <= 4096 (FLEXQ_ERR_UNSUPPORTED beyond) and
 * 0 < sparsity <= FLT_MAX (FLEXQ_ERR_INVALID otherwise).  Kept scores are decided
 * in fp32, as computed by the kernel. */
int flexq_attn_decode_kv4_topk(const uint16_t* qkv, int32_t B, int32_t b0, int32_t pos,
                               const flexq_kv4_layer* kv, float sparsity, uint16_t* out,
                               hipStream_t stream);

/* Decode attention on the host CPU over a 4-bit cache in HOST memory (source notes
 * "Flex Opt": the cpu_cache_compute policy and the load_cache path that attends in
 * a CPU workspace; "Pytorch Backend": mha_gen over a compressed cache dequantized
 * to fp32).  For caches too large for HBM: only the new token's q, k, v and the
 * output cross the host link.  Same arithmetic contract as flexq_attn_decode_kv4
 * (quantize-append at pos with the same code decisions, bit for bit; positions
 * [pad, pos]; fp32 scores and softmax; fp16 output).  Every pointer is a HOST
 * pointer: qkv fp16 [B][3h], out fp16 [B][h], and all arrays of kv (pad included).
 * Runs synchronously on `threads` host threads (<= 0: one per hardware thread),
 * one (sequence, head) pair per thread at a time, so results do not depend on the
 * thread count; returns when done.  No stream, no GPU.  Returns FLEXQ_ERR_DEVICE,
 * before touching the cache, if the host cannot allocate the threads' score
 * scratch (nthreads x (pos + 1) floats); fewer threads than asked run the same work. */
int flexq_host_attn_decode_kv4(const uint16_t* qkv, int32_t B, int32_t b0, int32_t pos,
                               const flexq_kv4_layer* kv, uint16_t* out, int32_t threads);

/* ---------------------------------------------------------------- model pieces
 * Token + position embedding (`opt_input_embed`, source notes "Pytorch Backend"):
 * out[m] = fp16(dequant(embed row tokens[m]) + pos[p + 2]) with position
 * p = max(pos_base + m % seq - pad[m / seq], 0) (prefill: pos_base 0, seq S; decode:
 * pos_base = pos, seq 1).  pad: NULL (no padding) or device int32 [n / seq], the
 * left padding of each sequence, so positions count from its first real token.
 * tokens: device int32 [n], ids outside [0, vocab) are clamped.
 * pos_base + min(n, seq) - 1 + 2 must be < pos_rows. */
int flexq_embed(const int32_t* tokens, int64_t n, int32_t pos_base, int32_t seq,
                const int32_t* pad, const flexq_w4* embed, const uint16_t* pos,
                int32_t pos_rows, uint16_t* out, hipStream_t stream);

/* Greedy pick: next[m] = argmax_n logits[m][n], lowest index among equal maxima. */
int flexq_argmax(const float* logits, int64_t M, int64_t N, int32_t* next, hipStream_t stream);

/* Next tokens of M sequences from fp32 logits [M][N] under a generation config
 * (see flexq_gen_config; gen is a HOST pointer, NULL = greedy).  Row m is sequence
 * m0 + m of generation step `step`; sampling needs 0 <= step < 65536 and
 * m0 + M <= 65536.  stopped: NULL, or device int32 [M] read and updated in place
 * (used only with a stop token).  next: device int32 [M].  Errors: bad sizes,
 * temperature <= 0 or not finite, stop >= N -> FLEXQ_ERR_INVALID. */
int flexq_pick(const float* logits, int64_t M, int64_t N, const flexq_gen_config* gen,
               int32_t step, int32_t m0, int32_t* stopped, int32_t* next, hipStream_t stream);

/* One decoder layer, prefill of nb sequences of S tokens: x_out [nb*S][h] from
 * x_in [nb*S][h] (distinct buffers), filling cache rows b0.. positions [0, S). */
size_t flexq_layer_workspace_size(int32_t hidden, int32_t heads, int32_t ffn, int64_t rows,
                                  int32_t max_len);
int flexq_prefill_layer(const flexq_layer* L, const flexq_kv4_layer* kv, int32_t hidden,
                        int32_t heads, int32_t ffn, const uint16_t* x_in, int32_t nb, int32_t S,
                        int32_t b0, uint16_t* x_out, void* ws, size_t ws_bytes,
                        hipStream_t stream);
/* One decoder layer, one decode step of B sequences at position pos. */
int flexq_decode_layer(const flexq_layer* L, const flexq_kv4_layer* kv, int32_t hidden,
                       int32_t heads, int32_t ffn, const uint16_t* x_in, int32_t B, int32_t b0,
                       int32_t pos, uint16_t* x_out, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* ---------------------------------------------------------------- whole model
 * Workspace for prefill micro-batches of up to max_prefill_rows = nb*S token
 * rows and decode batches of up to max_batch sequences with caches of max_len. */
size_t flexq_model_workspace_size(int32_t hidden, int32_t heads, int32_t ffn, int32_t vocab,
                                  int64_t max_prefill_rows, int32_t max_batch, int32_t max_len);

/* Prefill of one micro-batch (source notes, "Flex Opt": embedding, layers, output
 * head): tokens int32 [nb][S] for cache rows b0..b0+nb-1.  Ragged prompts are
 * left-padded to S; the pad counts are kv[0].pad (every layer's kv must point at
 * the same array, rows b0.. written before the call), used for the positions and
 * by every layer's attention.  Writes the first
 * generated token of each sequence to next [nb] and, if logits != NULL, the fp32
 * logits of the last prompt position to logits [nb][vocab]. */
int flexq_prefill(const flexq_model* m, const int32_t* tokens, int32_t nb, int32_t S, int32_t b0,
                  int32_t* next, float* logits, hipStream_t stream);

/* One decode step of B sequences (walkthrough section 4.1, `generate`: after the
 * prompt, each step feeds every sequence's last token through the model and picks
 * the next; source notes "Flex Opt": per step the engine walks the layers, loading
 * and storing each layer's cache around its compute).  Cache rows 0..B-1: tokens
 * int32 [B] at position pos -> next [B] (and logits [B][vocab] if not NULL).  The
 * token is embedded at position pos - pad of its row, each layer appends its k, v at
 * cache position pos (quantized) and attends over [pad, pos].  Without a
 * host tier the call neither synchronises nor allocates, so a caller may capture
 * it in a HIP graph (pos and the generation config are baked into the captured
 * kernels); with host rows it waits on the stream once per layer (see
 * flexq_host_tier).  Errors: B beyond the caches, pos >= max_len, a too small
 * host staging area -> FLEXQ_ERR_INVALID; sparse attention with a host tier ->
 * FLEXQ_ERR_UNSUPPORTED. */
int flexq_decode_step(const flexq_model* m, const int32_t* tokens, int32_t B, int32_t pos,
                      int32_t* next, float* logits, hipStream_t stream);

/* ---------------------------------------------------------------- measurement aid
 * Not part of the decoder path: the sustained rate of the fp16 matrix cores, the
 * ceiling the GEMMs are measured against.  `blocks` work-groups of 256 threads (two
 * per CU) each stream 4 * iters v_mfma_f32_32x32x16_f16 per wave (32768 flop each)
 * on independent accumulators; mode 0 constant operands, 1 fixed pseudo-random fp16
 * operands, 2 the same with their mantissa bits changed every iteration.  out: device
 * float [blocks * 256] (a checksum per thread).  Bad arguments -> FLEXQ_ERR_INVALID. */
int flexq_probe_mfma(int32_t mode, int32_t blocks, int32_t iters, float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* FLEXQ_H */
