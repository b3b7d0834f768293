// Decoder-layer and whole-model sequencing on one stream (source notes, "Flex
// Opt": an OPT model is an embedding, N transformer layers and an output head;
// per layer the engine runs compute_layer between cache loads/stores).
//
// With every tensor resident in HBM a layer is a fixed chain of kernel launches on
// the caller's stream with no host synchronisation (a host-DRAM cache tier adds one
// wait per decode layer, for the CPU's share of the attention):
//   LN1 -> QKV linear (+bias) -> attention (prefill: causal MFMA + KV4 store,
//   decode: KV4 append + split-K) -> out linear (+bias, +residual) -> LN2 ->
//   FC1 (+bias, ReLU) -> FC2 (+bias, +residual).
// Scratch comes from the caller's workspace, carved into 256-byte aligned slices.
#include <algorithm>

#include "common.h"
#include "pick.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Carve {
  char* base;
  size_t used, cap;
  void* take(size_t bytes) {
    void* p = base ? base + used : nullptr;
    used += align_up(bytes);
    return p;
  }
};

size_t gemm_ws(int64_t rows, int32_t h, int32_t ffn) {
  size_t w = 0;
  w = std::max(w, flexq_linear_w4_workspace_size(rows, 3 * (int64_t)h, h));
  w = std::max(w, flexq_linear_w4_workspace_size(rows, h, h));
  w = std::max(w, flexq_linear_w4_workspace_size(rows, ffn, h));
  w = std::max(w, flexq_linear_w4_workspace_size(rows, h, ffn));
  return w;
}

struct LayerScratch {
  uint16_t *a, *qkv, *attn, *x1, *u;
  void* ws;
  size_t ws_bytes;
};

// Lays out (or, with base == nullptr, sizes) the scratch of one layer call.
size_t layer_carve(char* base, int32_t h, int32_t heads, int32_t ffn, int64_t rows,
                   int32_t max_len, LayerScratch* s) {
  Carve c{base, 0, 0};
  LayerScratch t;
  t.a = (uint16_t*)c.take((size_t)rows * h * 2);
  t.qkv = (uint16_t*)c.take((size_t)rows * 3 * h * 2);
  t.attn = (uint16_t*)c.take((size_t)rows * h * 2);
  t.x1 = (uint16_t*)c.take((size_t)rows * h * 2);
  t.u = (uint16_t*)c.take((size_t)rows * ffn * 2);
  const int32_t hd = heads > 0 ? h / heads : 0;
  size_t ws = gemm_ws(rows, h, ffn);
  if (rows <= 0x7FFFFFFF && max_len > 0)
    ws = std::max(ws, flexq_attn_decode_workspace_size((int32_t)rows, heads, hd, max_len - 1));
  t.ws = c.take(ws);
  t.ws_bytes = ws;
  if (s) *s = t;
  return c.used;
}

int check_layer_args(const flexq_layer* L, const flexq_kv4_layer* kv, int32_t h, int32_t heads,
                     int32_t ffn) {
  if (!L || !kv || h <= 0 || heads <= 0 || ffn <= 0 || h % heads) return FLEXQ_ERR_INVALID;
  if (kv->heads != heads || kv->head_dim != h / heads) return FLEXQ_ERR_INVALID;
  if (L->wqkv.rows != 3 * (int64_t)h || L->wqkv.cols != h || L->wo.rows != h || L->wo.cols != h ||
      L->w1.rows != ffn || L->w1.cols != h || L->w2.rows != h || L->w2.cols != ffn)
    return FLEXQ_ERR_INVALID;
  if (!L->ln1_g || !L->ln1_b || !L->ln2_g || !L->ln2_b || !L->bqkv || !L->bo || !L->b1 || !L->b2)
    return FLEXQ_ERR_INVALID;
  return FLEXQ_OK;
}

#define TRY(expr)                       \
  do {                                  \
    const int _st = (expr);             \
    if (_st != FLEXQ_OK) return _st;    \
  } while (0)

// Brackets one linear layer's launches with the caller's trace events, if any.
struct TraceScope {
  flexq_trace* t;
  hipStream_t s;
  int slot;
  TraceScope(flexq_trace* tr, hipStream_t st, int kind, int64_t rows) : t(tr), s(st), slot(-1) {
    if (t && t->events && t->count < t->capacity) {
      slot = t->count++;
      if (t->kinds) t->kinds[slot] = kind;
      if (t->rows) t->rows[slot] = rows;
      (void)hipEventRecord(t->events[2 * slot], s);
    }
  }
  ~TraceScope() {
    if (slot >= 0) (void)hipEventRecord(t->events[2 * slot + 1], s);
  }
};

// Decode rows >= row0 whose cache is in host memory: their attention runs on the CPU.
struct HostSplit {
  const flexq_kv4_layer* kv;  // this layer's host cache
  int32_t row0, threads;
  uint16_t *qkv, *out;        // pinned host staging
};

int run_layer(const flexq_layer* L, const flexq_kv4_layer* kv, int32_t h,
              const uint16_t* x_in, int64_t rows, bool prefill, int32_t nb, int32_t S,
              int32_t b0, int32_t pos, uint16_t* x_out, const LayerScratch& s,
              hipStream_t stream, flexq_trace* tr = nullptr, float sparsity = 0.0f,
              const HostSplit* hs = nullptr) {
  TRY(flexq_layernorm(x_in, rows, h, h, L->ln1_g, L->ln1_b, s.a, stream));
  {
    TraceScope ts(tr, stream, FLEXQ_TRACE_QKV, rows);
    TRY(flexq_linear_w4(s.a, rows, &L->wqkv, L->bqkv, nullptr, 0, s.qkv, s.ws, s.ws_bytes, stream));
  }
  if (prefill) {
    TRY(flexq_attn_prefill(s.qkv, nb, S, b0, kv, s.attn, stream));
  } else {
    const int32_t nd = hs ? std::min(nb, hs->row0) : nb;  // rows with a device cache
    const int32_t nhost = nb - nd;
    if (nhost > 0) {  // the host rows' q, k, v must be in host memory before the CPU starts
      if (hipMemcpyAsync(hs->qkv, s.qkv + (size_t)nd * 3 * h, (size_t)nhost * 3 * h * 2,
                         hipMemcpyDeviceToHost, stream) != hipSuccess ||
          hipStreamSynchronize(stream) != hipSuccess)
        return FLEXQ_ERR_DEVICE;
    }
    if (nd > 0) {  // enqueued first, so the GPU attends while the CPU does
      if (sparsity > 0.0f && sparsity < 1.0f)
        TRY(flexq_attn_decode_kv4_topk(s.qkv, nd, b0, pos, kv, sparsity, s.attn, stream));
      else
        TRY(flexq_attn_decode_kv4(s.qkv, nd, b0, pos, kv, s.attn, s.ws, s.ws_bytes, stream));
    }
    if (nhost > 0) {
      TRY(flexq_host_attn_decode_kv4(hs->qkv, nhost, 0, pos, hs->kv, hs->out, hs->threads));
      if (hipMemcpyAsync(s.attn + (size_t)nd * h, hs->out, (size_t)nhost * h * 2,
                         hipMemcpyHostToDevice, stream) != hipSuccess)
        return FLEXQ_ERR_DEVICE;
    }
  }
  {
    TraceScope ts(tr, stream, FLEXQ_TRACE_OUT, rows);
    TRY(flexq_linear_w4(s.attn, rows, &L->wo, L->bo, x_in, 0, s.x1, s.ws, s.ws_bytes, stream));
  }
  TRY(flexq_layernorm(s.x1, rows, h, h, L->ln2_g, L->ln2_b, s.a, stream));
  {
    TraceScope ts(tr, stream, FLEXQ_TRACE_FC1, rows);
    TRY(flexq_linear_w4(s.a, rows, &L->w1, L->b1, nullptr, 1, s.u, s.ws, s.ws_bytes, stream));
  }
  {
    TraceScope ts(tr, stream, FLEXQ_TRACE_FC2, rows);
    TRY(flexq_linear_w4(s.u, rows, &L->w2, L->b2, s.x1, 0, x_out, s.ws, s.ws_bytes, stream));
  }
  return FLEXQ_OK;
}

struct ModelScratch {
  uint16_t *x0, *x1, *lnf;
  float* logits;
  char* layer_base;
  size_t layer_bytes;
  void* head_ws;
  size_t head_ws_bytes;
};

size_t model_carve(char* base, int32_t h, int32_t heads, int32_t ffn, int32_t vocab,
                   int64_t max_rows, int32_t max_batch, int32_t max_len, ModelScratch* s) {
  Carve c{base, 0, 0};
  ModelScratch t;
  const int64_t rows = std::max<int64_t>(max_rows, max_batch);
  t.x0 = (uint16_t*)c.take((size_t)rows * h * 2);
  t.x1 = (uint16_t*)c.take((size_t)rows * h * 2);
  t.lnf = (uint16_t*)c.take((size_t)max_batch * h * 2);
  t.logits = (float*)c.take((size_t)max_batch * vocab * 4);
  t.head_ws_bytes = flexq_linear_w4_workspace_size(max_batch, vocab, h);
  t.head_ws = c.take(t.head_ws_bytes);
  t.layer_bytes = layer_carve(nullptr, h, heads, ffn, rows, max_len, nullptr);
  t.layer_base = (char*)c.take(t.layer_bytes);
  if (s) *s = t;
  return c.used;
}

// Validates the model's tap against a call of `rows` rows.
int check_tap(const flexq_model* m, int64_t rows) {
  const flexq_tap* t = m->tap;
  if (!t || t->count == 0) return FLEXQ_OK;
  if (t->count < 0 || !t->layers || !t->x || rows > t->rows_cap) return FLEXQ_ERR_INVALID;
  for (int i = 0; i < t->count; ++i)
    if (t->layers[i] < 0 || t->layers[i] > m->layers || !t->x[i]) return FLEXQ_ERR_INVALID;
  return FLEXQ_OK;
}

// Copies the hidden state x (rows x hidden) entering layer l (l == layers: the
// output head) into every tap buffer that names l.
int tap_copy(const flexq_model* m, int l, const uint16_t* x, int64_t rows, hipStream_t stream) {
  const flexq_tap* t = m->tap;
  if (!t) return FLEXQ_OK;
  for (int i = 0; i < t->count; ++i)
    if (t->layers[i] == l &&
        hipMemcpyAsync(t->x[i], x, (size_t)rows * m->hidden * 2, hipMemcpyDeviceToDevice,
                       stream) != hipSuccess)
      return FLEXQ_ERR_DEVICE;
  return FLEXQ_OK;
}

int check_model(const flexq_model* m) {
  if (!m || m->layers <= 0 || !m->layer || !m->kv || !m->pos || !m->lnf_g || !m->lnf_b)
    return FLEXQ_ERR_INVALID;
  if (m->embed.rows != m->vocab || m->embed.cols != m->hidden || !m->workspace)
    return FLEXQ_ERR_INVALID;
  if (const flexq_host_tier* t = m->host) {
    if (!t->kv || t->row0 < 0 || t->row0 > m->kv[0].batch) return FLEXQ_ERR_INVALID;
    if (m->attn_sparsity > 0.0f && m->attn_sparsity < 1.0f) return FLEXQ_ERR_UNSUPPORTED;
    for (int l = 0; l < m->layers; ++l)
      if (t->kv[l].heads != m->heads || t->kv[l].head_dim != m->hidden / m->heads ||
          t->kv[l].batch != t->kv[0].batch || t->kv[l].max_len != t->kv[0].max_len)
        return FLEXQ_ERR_INVALID;
  }
  return FLEXQ_OK;
}

// The device staging copy of one host micro-batch's K/V: nb rows laid out as a cache.
flexq_kv4_layer stage_view(const flexq_model* m, int32_t nb, int32_t b0) {
  const flexq_host_tier* t = m->host;
  const int32_t hd = m->hidden / m->heads;
  const size_t codes = (size_t)nb * m->heads * t->kv[0].max_len * (hd / 2);
  const size_t params = (size_t)nb * m->heads * t->kv[0].max_len * (hd / 64) * 2;  // fp16s
  char* p = (char*)t->stage;
  flexq_kv4_layer v;
  v.k_codes = (uint8_t*)p;
  v.v_codes = (uint8_t*)(p + codes);
  v.k_params = (uint16_t*)(p + 2 * codes);
  v.v_params = (uint16_t*)(p + 2 * codes + params * 2);
  v.batch = nb;
  v.heads = m->heads;
  v.head_dim = hd;
  v.max_len = t->kv[0].max_len;
  v.pad = m->kv[0].pad ? m->kv[0].pad + b0 : nullptr;
  return v;
}

// Copies the staged rows into host cache rows [r0, r0 + nb) of one layer.
int stage_to_host(const flexq_kv4_layer& st, const flexq_kv4_layer& hk, int32_t r0,
                  hipStream_t stream) {
  const size_t per_row_codes = (size_t)st.heads * st.max_len * (st.head_dim / 2);
  const size_t per_row_params = (size_t)st.heads * st.max_len * (st.head_dim / 64) * 2;
  const size_t nc = per_row_codes * st.batch, np = per_row_params * st.batch;
  if (hipMemcpyAsync(hk.k_codes + per_row_codes * r0, st.k_codes, nc, hipMemcpyDeviceToHost,
                     stream) != hipSuccess ||
      hipMemcpyAsync(hk.v_codes + per_row_codes * r0, st.v_codes, nc, hipMemcpyDeviceToHost,
                     stream) != hipSuccess ||
      hipMemcpyAsync(hk.k_params + per_row_params * r0, st.k_params, np * 2,
                     hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipMemcpyAsync(hk.v_params + per_row_params * r0, st.v_params, np * 2,
                     hipMemcpyDeviceToHost, stream) != hipSuccess)
    return FLEXQ_ERR_DEVICE;
  return FLEXQ_OK;
}

}  // namespace

extern "C" size_t flexq_host_stage_size(int32_t heads, int32_t head_dim, int32_t nb,
                                        int32_t max_len) {
  if (heads <= 0 || nb <= 0 || max_len <= 0 || (head_dim != 64 && head_dim != 128)) return 0;
  return (size_t)nb * heads * max_len * (head_dim / 2 + (head_dim / 64) * 4) * 2;
}

extern "C" size_t flexq_layer_workspace_size(int32_t hidden, int32_t heads, int32_t ffn,
                                             int64_t rows, int32_t max_len) {
  if (hidden <= 0 || heads <= 0 || ffn <= 0 || rows <= 0) return 0;
  return layer_carve(nullptr, hidden, heads, ffn, rows, max_len, nullptr);
}

extern "C" int flexq_prefill_layer(const flexq_layer* L, const flexq_kv4_layer* kv, int32_t hidden,
                                   int32_t heads, int32_t ffn, const uint16_t* x_in, int32_t nb,
                                   int32_t S, int32_t b0, uint16_t* x_out, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  TRY(check_layer_args(L, kv, hidden, heads, ffn));
  if (nb < 0 || S < 0 || b0 < 0 || !x_in || !x_out || x_in == x_out) return FLEXQ_ERR_INVALID;
  if (nb == 0 || S == 0) return FLEXQ_OK;
  const int64_t rows = (int64_t)nb * S;
  LayerScratch s;
  const size_t need = layer_carve((char*)ws, hidden, heads, ffn, rows, 0, &s);
  if (!ws || ws_bytes < need) return FLEXQ_ERR_INVALID;
  return run_layer(L, kv, hidden, x_in, rows, true, nb, S, b0, 0, x_out, s, stream);
}

extern "C" int flexq_decode_layer(const flexq_layer* L, const flexq_kv4_layer* kv, int32_t hidden,
                                  int32_t heads, int32_t ffn, const uint16_t* x_in, int32_t B,
                                  int32_t b0, int32_t pos, uint16_t* x_out, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  TRY(check_layer_args(L, kv, hidden, heads, ffn));
  if (B < 0 || b0 < 0 || pos < 0 || !x_in || !x_out || x_in == x_out) return FLEXQ_ERR_INVALID;
  if (B == 0) return FLEXQ_OK;
  LayerScratch s;
  const size_t need = layer_carve((char*)ws, hidden, heads, ffn, B, pos + 1, &s);
  if (!ws || ws_bytes < need) return FLEXQ_ERR_INVALID;
  return run_layer(L, kv, hidden, x_in, B, false, B, 1, b0, pos, x_out, s, stream);
}

extern "C" size_t flexq_model_workspace_size(int32_t hidden, int32_t heads, int32_t ffn,
                                             int32_t vocab, int64_t max_prefill_rows,
                                             int32_t max_batch, int32_t max_len) {
  if (hidden <= 0 || heads <= 0 || ffn <= 0 || vocab <= 0 || max_batch <= 0) return 0;
  return model_carve(nullptr, hidden, heads, ffn, vocab, max_prefill_rows, max_batch, max_len,
                     nullptr);
}

// Carves the model workspace for the rows, batch and context of one call; nothing
// in it outlives the call.
static int model_scratch(const flexq_model* m, int64_t rows, int32_t batch, int32_t max_len,
                         ModelScratch* s) {
  const size_t need = model_carve(nullptr, m->hidden, m->heads, m->ffn, m->vocab, rows, batch,
                                  max_len, nullptr);
  if (m->workspace_bytes < need) return FLEXQ_ERR_INVALID;
  model_carve((char*)m->workspace, m->hidden, m->heads, m->ffn, m->vocab, rows, batch, max_len, s);
  return FLEXQ_OK;
}

// Final LayerNorm, tied LM head and the token choice for cache rows b0 .. b0+nb-1
// whose logits follow position `step`; `fresh` at prefill (a sequence's first token).
static int model_head(const flexq_model* m, const uint16_t* x_last, int64_t stride, int32_t nb,
                      int32_t b0, int32_t step, bool fresh, int32_t* next, float* logits,
                      const ModelScratch& s, hipStream_t stream) {
  TRY(flexq_layernorm(x_last, nb, m->hidden, stride, m->lnf_g, m->lnf_b, s.lnf, stream));
  float* lg = logits ? logits : s.logits;
  {
    TraceScope ts(m->trace, stream, FLEXQ_TRACE_HEAD, nb);
    TRY(flexq_linear_w4_f32(s.lnf, nb, &m->embed, lg, s.head_ws, s.head_ws_bytes, stream));
  }
  TRY(flexq::launch_pick(lg, nb, m->vocab, m->gen, step, b0, m->stopped ? m->stopped + b0 : nullptr,
                  fresh, next, stream));
  return FLEXQ_OK;
}

extern "C" int flexq_prefill(const flexq_model* m, const int32_t* tokens, int32_t nb, int32_t S,
                             int32_t b0, int32_t* next, float* logits, hipStream_t stream) {
  TRY(check_model(m));
  if (nb < 0 || S < 0 || b0 < 0 || !tokens || !next) return FLEXQ_ERR_INVALID;
  if (nb == 0 || S == 0) return FLEXQ_OK;
  // cache rows (pad counts and stopped flags are indexed by them before any layer runs)
  const flexq_host_tier* ht = m->host;
  const bool host_rows = ht && b0 >= ht->row0;
  if (host_rows) {
    if ((int64_t)b0 - ht->row0 + nb > ht->kv[0].batch || S > ht->kv[0].max_len)
      return FLEXQ_ERR_INVALID;
    if (!ht->stage || ht->stage_bytes < flexq_host_stage_size(m->heads, m->hidden / m->heads, nb,
                                                              ht->kv[0].max_len))
      return FLEXQ_ERR_INVALID;
  } else if ((int64_t)b0 + nb > m->kv[0].batch || S > m->kv[0].max_len) {
    return FLEXQ_ERR_INVALID;   // also a micro-batch that straddles the host tier
  }
  const int64_t rows = (int64_t)nb * S;
  TRY(check_tap(m, rows));
  ModelScratch s;
  TRY(model_scratch(m, rows, nb, 0, &s));
  const int32_t* pad = m->kv[0].pad;
  TRY(flexq_embed(tokens, rows, 0, S, pad ? pad + b0 : nullptr, &m->embed, m->pos, m->pos_rows,
                  s.x0, stream));
  LayerScratch ls;
  layer_carve(s.layer_base, m->hidden, m->heads, m->ffn, rows, 0, &ls);
  uint16_t* x = s.x0;
  uint16_t* y = s.x1;
  const flexq_kv4_layer stage = host_rows ? stage_view(m, nb, b0) : flexq_kv4_layer{};
  for (int l = 0; l < m->layers; ++l) {
    TRY(check_layer_args(&m->layer[l], &m->kv[l], m->hidden, m->heads, m->ffn));
    TRY(tap_copy(m, l, x, rows, stream));
    if (host_rows) {  // K/V through the device stage, then to the host tier
      TRY(run_layer(&m->layer[l], &stage, m->hidden, x, rows, true, nb, S, 0, 0, y, ls,
                    stream, m->trace));
      TRY(stage_to_host(stage, ht->kv[l], b0 - ht->row0, stream));
    } else {
      TRY(run_layer(&m->layer[l], &m->kv[l], m->hidden, x, rows, true, nb, S, b0, 0, y,
                    ls, stream, m->trace));
    }
    std::swap(x, y);
  }
  TRY(tap_copy(m, m->layers, x, rows, stream));
  return model_head(m, x + (int64_t)(S - 1) * m->hidden, (int64_t)S * m->hidden, nb, b0, S - 1,
                    true, next, logits, s, stream);
}

extern "C" int flexq_decode_step(const flexq_model* m, const int32_t* tokens, int32_t B,
                                 int32_t pos, int32_t* next, float* logits, hipStream_t stream) {
  TRY(check_model(m));
  if (B < 0 || pos < 0 || !tokens || !next) return FLEXQ_ERR_INVALID;
  if (B == 0) return FLEXQ_OK;
  const flexq_host_tier* ht = m->host;
  const int32_t nhost = ht ? std::max(0, B - ht->row0) : 0;
  if (B - nhost > m->kv[0].batch || pos >= m->kv[0].max_len) return FLEXQ_ERR_INVALID;
  if (nhost > 0) {
    if (nhost > ht->kv[0].batch || pos >= ht->kv[0].max_len) return FLEXQ_ERR_INVALID;
    if (!ht->host_ws || ht->host_ws_bytes < (size_t)nhost * 4 * m->hidden * 2)
      return FLEXQ_ERR_INVALID;
  }
  TRY(check_tap(m, B));
  ModelScratch s;
  TRY(model_scratch(m, B, B, pos + 1, &s));
  TRY(flexq_embed(tokens, B, pos, 1, m->kv[0].pad, &m->embed, m->pos, m->pos_rows, s.x0,
                  stream));
  LayerScratch ls;
  layer_carve(s.layer_base, m->hidden, m->heads, m->ffn, B, pos + 1, &ls);
  uint16_t* x = s.x0;
  uint16_t* y = s.x1;
  for (int l = 0; l < m->layers; ++l) {
    TRY(check_layer_args(&m->layer[l], &m->kv[l], m->hidden, m->heads, m->ffn));
    TRY(tap_copy(m, l, x, B, stream));
    HostSplit hs{};
    if (nhost > 0)
      hs = HostSplit{&ht->kv[l], ht->row0, ht->threads, (uint16_t*)ht->host_ws,
                     (uint16_t*)ht->host_ws + (size_t)nhost * 3 * m->hidden};
    TRY(run_layer(&m->layer[l], &m->kv[l], m->hidden, x, B, false, B, 1, 0, pos, y, ls,
                  stream, m->trace, m->attn_sparsity, nhost > 0 ? &hs : nullptr));
    std::swap(x, y);
  }
  TRY(tap_copy(m, m->layers, x, B, stream));
  return model_head(m, x, m->hidden, B, 0, pos, false, next, logits, s, stream);
}
