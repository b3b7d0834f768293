// Decode attention on the host CPU over a 4-bit KV cache held in host memory: the
// pages' CPU-side cache compute (source notes, section "Flex Opt": the
// cpu_cache_compute policy, and the load_cache path that computes attention in a CPU
// workspace; "Pytorch Backend": mha_gen over a compressed cache decompressed into an
// fp32 workspace).  Only q, k, v of the new token and the attention output cross the
// host link; the cache never does.
//
// Same contract as the GPU decode attention: the new token's k and v are quantized
// into position pos (group 64, 4 bits, the fp32 decision sequence of the walkthrough's
// section 6.3 as every quantizer here uses it), then positions [pad, pos] are read
// back, dequantized to fp32 and attended with an fp32 softmax; fp16 output.
//
// Work is split over (sequence, head) pairs, round-robin over the threads, each pair
// computed by one thread alone, so the result does not depend on the thread count.
// This file is compiled for the host only (x86-64 with AVX2 and FMA), with implicit
// floating-point contraction off: the quantizer's code decisions must not see fused
// multiply-adds; the attention sums use explicit FMA intrinsics.
#include <immintrin.h>

#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "flexq.h"

namespace {

inline float h2f(uint16_t b) {
  _Float16 h;
  std::memcpy(&h, &b, 2);
  return (float)h;
}

inline uint16_t f2h(float f) {
  const _Float16 h = (_Float16)f;  // round to nearest even
  uint16_t b;
  std::memcpy(&b, &h, 2);
  return b;
}

// One 64-element group of fp16 values -> 32 code bytes and (offset, scale) as fp16 bits:
// step = fp16(fl32(max - min) / 15) (0 for a constant group, 2^-24 if it underflows),
// code = clamp(rne(fl32(x - min) * fl32(1 / step)), 0, 15), offset = min (+0 for 0).
void quantize_group(const uint16_t* x, uint8_t* codes, uint16_t* param) {
  float v[64];
  for (int i = 0; i < 64; ++i) v[i] = h2f(x[i]);
  float mn = v[0], mx = v[0];
  for (int i = 1; i < 64; ++i) {
    mn = std::fmin(mn, v[i]);
    mx = std::fmax(mx, v[i]);
  }
  const bool constant = mx == mn;
  const float r = mx - mn;
  uint16_t s16 = f2h(r / 15.0f);
  if (constant) s16 = 0;
  else if (s16 == 0) s16 = 0x0001;  // 2^-24
  const float inv = constant ? 0.0f : 1.0f / h2f(s16);
  for (int j = 0; j < 32; ++j) {
    uint32_t c[2];
    for (int e = 0; e < 2; ++e) {
      float t = (v[2 * j + e] - mn) * inv;
      t = std::fmin(std::fmax(t, 0.0f), 15.0f);
      c[e] = (uint32_t)std::nearbyint(t);  // default rounding: to nearest even
    }
    codes[j] = (uint8_t)(c[0] | (c[1] << 4));
  }
  param[0] = f2h(mn == 0.0f ? 0.0f : mn);
  param[1] = s16;
}

struct Job {
  const uint16_t* qkv;
  int B, b0, pos;
  const flexq_kv4_layer* kv;
  uint16_t* out;
};

// AVX2 helpers.  Code byte i of a group holds element 2i (low nibble) and 2i+1 (high
// nibble); q and the accumulators are kept split the same way (even / odd elements),
// 8 floats per vector, so no shuffle is needed per position.
struct Nibbles {
  __m256 lo[4], hi[4];  // lo[j][e] = code of element 2 (8j + e), hi: element 2 (8j + e) + 1
};

inline void load_codes(const uint8_t* c, Nibbles& n) {
  const __m128i m = _mm_set1_epi8(0x0F);
  for (int half = 0; half < 2; ++half) {
    const __m128i x = _mm_loadu_si128((const __m128i*)(c + 16 * half));
    const __m128i l = _mm_and_si128(x, m);
    const __m128i h = _mm_and_si128(_mm_srli_epi16(x, 4), m);
    n.lo[2 * half] = _mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(l));
    n.lo[2 * half + 1] = _mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(_mm_srli_si128(l, 8)));
    n.hi[2 * half] = _mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(h));
    n.hi[2 * half + 1] = _mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(_mm_srli_si128(h, 8)));
  }
}

// Sum of the 8 lanes in a fixed order.
inline float hsum(__m256 v) {
  const __m128 s = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
  const __m128 t = _mm_add_ps(s, _mm_movehl_ps(s, s));
  return _mm_cvtss_f32(_mm_add_ss(t, _mm_shuffle_ps(t, t, 1)));
}

// Attention of one (sequence, head) pair; scratch holds max_len + 1 floats.
void attend(const Job& J, int bi, int head, float* sc) {
  const flexq_kv4_layer& kv = *J.kv;
  const int hd = kv.head_dim, G = hd / 64, h = kv.heads * hd;
  const uint16_t* row = J.qkv + (size_t)bi * 3 * h;
  const size_t slot0 = ((size_t)(J.b0 + bi) * kv.heads + head) * (size_t)kv.max_len;
  // 1. quantize-append of the new k and v
  for (int g = 0; g < G; ++g) {
    const size_t at = (slot0 + J.pos) * G + g;
    quantize_group(row + h + head * hd + 64 * g, kv.k_codes + at * 32, kv.k_params + at * 2);
    quantize_group(row + 2 * h + head * hd + 64 * g, kv.v_codes + at * 32, kv.v_params + at * 2);
  }
  int npad = kv.pad ? kv.pad[J.b0 + bi] : 0;
  npad = npad < 0 ? 0 : (npad > J.pos ? J.pos : npad);
  // q split into even / odd elements per group, and its per-group sum
  __m256 qe[2][4], qo[2][4];
  float qsum[2];
  for (int g = 0; g < G; ++g) {
    alignas(32) float e[32], o[32];
    for (int i = 0; i < 32; ++i) {
      e[i] = h2f(row[head * hd + 64 * g + 2 * i]);
      o[i] = h2f(row[head * hd + 64 * g + 2 * i + 1]);
    }
    __m256 s = _mm256_setzero_ps();
    for (int j = 0; j < 4; ++j) {
      qe[g][j] = _mm256_load_ps(e + 8 * j);
      qo[g][j] = _mm256_load_ps(o + 8 * j);
      s = _mm256_add_ps(s, _mm256_add_ps(qe[g][j], qo[g][j]));
    }
    qsum[g] = hsum(s);
  }
  const float scale = 1.0f / std::sqrt((float)hd);
  Nibbles n;
  // 2. scores: sum over groups of step * (q . codes) + offset * sum(q)
  float mx = -INFINITY;
  for (int t = npad; t <= J.pos; ++t) {
    const size_t at = (slot0 + t) * G;
    float acc = 0.0f;
    for (int g = 0; g < G; ++g) {
      load_codes(kv.k_codes + (at + g) * 32, n);
      __m256 d = _mm256_mul_ps(qe[g][0], n.lo[0]);
      d = _mm256_fmadd_ps(qo[g][0], n.hi[0], d);
      for (int j = 1; j < 4; ++j) {
        d = _mm256_fmadd_ps(qe[g][j], n.lo[j], d);
        d = _mm256_fmadd_ps(qo[g][j], n.hi[j], d);
      }
      const float off = h2f(kv.k_params[(at + g) * 2]), st = h2f(kv.k_params[(at + g) * 2 + 1]);
      acc += st * hsum(d) + off * qsum[g];
    }
    sc[t] = acc * scale;
    mx = std::fmax(mx, sc[t]);
  }
  // 3. softmax
  float sum = 0.0f;
  for (int t = npad; t <= J.pos; ++t) {
    sc[t] = std::exp(sc[t] - mx);
    sum += sc[t];
  }
  // 4. o = sum_t p_t (step_t * codes_t + offset_t): the step part per lane, the offset
  // part as one scalar per group
  __m256 oe[2][4], oo[2][4];
  float pm[2] = {0.0f, 0.0f};
  for (int g = 0; g < G; ++g)
    for (int j = 0; j < 4; ++j) oe[g][j] = oo[g][j] = _mm256_setzero_ps();
  for (int t = npad; t <= J.pos; ++t) {
    const size_t at = (slot0 + t) * G;
    const float p = sc[t];
    for (int g = 0; g < G; ++g) {
      load_codes(kv.v_codes + (at + g) * 32, n);
      const float off = h2f(kv.v_params[(at + g) * 2]), st = h2f(kv.v_params[(at + g) * 2 + 1]);
      const __m256 ps = _mm256_set1_ps(p * st);
      pm[g] += p * off;
      for (int j = 0; j < 4; ++j) {
        oe[g][j] = _mm256_fmadd_ps(ps, n.lo[j], oe[g][j]);
        oo[g][j] = _mm256_fmadd_ps(ps, n.hi[j], oo[g][j]);
      }
    }
  }
  const float inv = 1.0f / sum;
  uint16_t* orow = J.out + (size_t)bi * h + head * hd;
  for (int g = 0; g < G; ++g) {
    alignas(32) float e[32], o[32];
    for (int j = 0; j < 4; ++j) {
      _mm256_store_ps(e + 8 * j, oe[g][j]);
      _mm256_store_ps(o + 8 * j, oo[g][j]);
    }
    for (int i = 0; i < 32; ++i) {
      orow[64 * g + 2 * i] = f2h((e[i] + pm[g]) * inv);
      orow[64 * g + 2 * i + 1] = f2h((o[i] + pm[g]) * inv);
    }
  }
}

}  // namespace

extern "C" int flexq_host_attn_decode_kv4(const uint16_t* qkv, int32_t B, int32_t b0,
                                          int32_t pos, const flexq_kv4_layer* kv, uint16_t* out,
                                          int32_t threads) {
  if (!kv || B < 0 || b0 < 0 || pos < 0) return FLEXQ_ERR_INVALID;
  if (B == 0) return FLEXQ_OK;
  if (!qkv || !out) return FLEXQ_ERR_INVALID;
  if (kv->head_dim != 64 && kv->head_dim != 128) return FLEXQ_ERR_UNSUPPORTED;
  if (kv->heads <= 0 || (int64_t)b0 + B > kv->batch || pos >= kv->max_len) return FLEXQ_ERR_INVALID;
  if (!kv->k_codes || !kv->v_codes || !kv->k_params || !kv->v_params) return FLEXQ_ERR_INVALID;
  const Job J{qkv, B, b0, pos, kv, out};
  const int64_t pairs = (int64_t)B * kv->heads;
  int nt = threads > 0 ? threads : (int)std::thread::hardware_concurrency();
  if (nt < 1) nt = 1;
  if (nt > pairs) nt = (int)pairs;
  // every allocation happens here, before any work starts, so nothing can throw
  // inside a worker and no exception leaves this function
  std::vector<float> scratch;
  std::vector<std::thread> pool;
  try {
    scratch.resize((size_t)nt * ((size_t)pos + 1));
    pool.reserve(nt - 1);
  } catch (...) {
    return FLEXQ_ERR_DEVICE;  // host memory exhausted
  }
  auto work = [&](int w) {
    float* sc = scratch.data() + (size_t)w * ((size_t)pos + 1);
    for (int64_t p = w; p < pairs; p += nt) attend(J, (int)(p / kv->heads), (int)(p % kv->heads), sc);
  };
  int started = 1;
  try {
    for (int w = 1; w < nt; ++w) {
      pool.emplace_back(work, w);
      ++started;
    }
  } catch (...) {  // the system gave fewer threads: this thread takes the other shares
  }
  for (int w = started; w < nt; ++w) work(w);
  work(0);
  for (auto& t : pool) t.join();
  return FLEXQ_OK;
}
