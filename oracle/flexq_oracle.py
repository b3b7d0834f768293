"""Oracle for the group-wise 4-bit weight + KV-cache OPT decoder path.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It is a plain, slow, obviously correct CPU
implementation written from the pages' description; it shares no code with the HIP
library and never calls it.

Sources (cited by title and section):
  [WALK]  "FlexGen 单 GPU 高吞吐大模型推理引擎：论文解读与源码实战指南" (FlexGen single-GPU
          high-throughput inference engine: paper reading and source walkthrough),
          section 6.3 (4-bit group-wise compression of weights and KV cache),
          section 5.1 (throughput table and definition), section 4.1 (generate API).
  [NOTES] "FlexGen" source notes (PtirisNote), sections "Flex Opt" (model = embedding,
          N transformer layers, output head; generate loop) and "Pytorch Backend"
          (mha for prefill, mha_gen for decode, opt_input_embed / opt_output_embed,
          compressed tensors stored as a triple, fp32 CPU workspace for attention).

Precision.  Floating point is evaluated in float64 (numpy, BLAS matmul as the
contraction primitive), and rounded to fp16 only where the pages keep fp16 tensors
(every layer input/output the engine stores).  The one exception is the quantizer:
its codes are integers decided by floating point, so it takes those decisions in
fp32, the precision of the kernel it checks (IEEE division, round-to-nearest-even,
no fused multiply-add), as a fixed sequence written out in `quantize`.

Readings of the pages where they leave a step open:
  * per group: offset = group minimum, scale = step = (max - min) / 15, both fp16;
    [WALK] section 6.3 names one fp16 "scale" tensor; an asymmetric (symmetric=False)
    code needs an offset as well, so the params hold the pair (offset, scale);
  * codes round half to even and are clamped to [0, 15];
  * constant group -> scale 0, all codes 0; a non-zero range whose step underflows
    fp16 gets the smallest fp16 subnormal 2^-24; a zero offset is stored as +0;
  * element 2j goes to the low nibble of byte j, element 2j+1 to the high nibble;
  * weights are [out][in] and grouped along `in` (group_dim 0 of the pages' config,
    the input dimension); KV entries are grouped along head_dim within one head
    (group_dim 2 of [B][heads][head_dim]-shaped caches);
  * dequantized weights are fp16 (the operand precision), dequantized KV values are
    exact (the pages decompress the cache into an fp32 workspace);
  * prefill attention reads the fp16 K/V it has just computed, then stores them 4-bit;
    decode attention reads every position, its own included, back from the 4-bit cache;
  * OPT layer: pre-LayerNorm (eps 1e-5), biases on all projections, ReLU FFN,
    1/sqrt(head_dim) applied to the score, learned positions with offset 2, final
    LayerNorm, LM head tied to the 4-bit token embedding without bias, greedy argmax
    with the lowest index winning ties;
  * sampling ([WALK] section 4.1 do_sample / temperature; [NOTES] "Flex Opt" Task and
    stopped flags): a draw from softmax(logits / T) taken by the Gumbel-max rule in
    float64, its uniforms from SplitMix64 (a counter-based generator, implemented on
    each side from its published definition) keyed by (seed, step, sequence, token);
    a sequence that produces the stop token is stopped and produces it from then on;
  * attention sparsity ([NOTES] "Flex Opt": the attn_sparsity policy, no mechanism
    given): in decode attention each query keeps its ceil(n * sparsity) highest scores
    (lower position first on equal scores) and takes the softmax over those alone;
    prefill attention stays dense;
  * ragged prompts ([NOTES] "Flex Opt": the attention_mask buffer of `generate`): prompts
    are left-padded to a common length; a sequence's pad count is kept with its cache
    row; attention never sees a pad key (a pad query's output is 0) and positions count
    from the first real token, so a padded sequence computes what it would alone.
"""
from __future__ import annotations

import numpy as np

GROUP = 64          # group_size of both CompressionConfigs in [WALK] section 6.3
BITS = 4            # num_bits
QMAX = (1 << BITS) - 1
LN_EPS = 1e-5
F16 = np.float16
F32 = np.float32
F64 = np.float64


# ----------------------------------------------------------------------------- packing

def pack_nibbles(c: np.ndarray) -> np.ndarray:
    """[..., n] codes in [0,15] -> [..., n/2] bytes; element 2j low nibble, 2j+1 high."""
    c = np.asarray(c, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """[..., n/2] bytes -> [..., n] codes (inverse of pack_nibbles)."""
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = b & 0x0F
    out[..., 1::2] = b >> 4
    return out


# ----------------------------------------------------------------------------- quantizer

def quantize(x) -> tuple[np.ndarray, np.ndarray]:
    """Group-wise asymmetric min/max 4-bit quantization ([WALK] section 6.3).

    x: fp16 [..., cols], cols a multiple of 64; groups are 64 consecutive elements
    of the innermost dimension.  Returns
      codes  uint8 [..., cols/2]       (num_groups * group_size/2 bytes, two codes a byte)
      params fp16  [..., cols/64, 2]   (offset, scale) per group.
    """
    x = np.asarray(x, dtype=F16)
    cols = x.shape[-1]
    if cols % GROUP:
        raise ValueError("grouped dimension must be a multiple of 64")
    g = x.reshape(x.shape[:-1] + (cols // GROUP, GROUP))
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    # step = (max - min) / 15, evaluated as fp32 subtract, fp32 divide, fp16 round
    r = mx.astype(F32) - mn.astype(F32)
    s = (r / F32(QMAX)).astype(F16)
    const = mx == mn
    s = np.where(const, F16(0), np.where(s == 0, F16(2.0 ** -24), s)).astype(F16)
    s32 = s.astype(F32)
    with np.errstate(divide="ignore"):
        inv = np.where(const, F32(0), F32(1) / np.where(const, F32(1), s32)).astype(F32)
    # codes: round((x - min) * (1/step)) half to even, clamp to [0, 15]
    t = (g.astype(F32) - mn[..., None].astype(F32)) * inv[..., None]
    c = np.clip(np.rint(t), 0, QMAX).astype(np.uint8)
    c[const] = 0
    offset = (mn.astype(F32) + F32(0)).astype(F16)     # stores a zero minimum as +0
    codes = pack_nibbles(c.reshape(x.shape))
    params = np.stack([offset, s], axis=-1).astype(F16)
    return codes, params


def _expand_params(params: np.ndarray, cols: int):
    off = np.repeat(params[..., 0].astype(F64), GROUP, axis=-1)
    scale = np.repeat(params[..., 1].astype(F64), GROUP, axis=-1)
    assert off.shape[-1] == cols
    return off, scale


def dequantize_exact(codes, params) -> np.ndarray:
    """code * scale + offset, exact (float64 holds it without rounding)."""
    c = unpack_nibbles(codes).astype(F64)
    off, scale = _expand_params(np.asarray(params, dtype=F16), c.shape[-1])
    return c * scale + off


def dequantize_weight(codes, params) -> np.ndarray:
    """Weights are decompressed back to fp16, the operand precision: one rounding."""
    return dequantize_exact(codes, params).astype(F16)


def dequantize_kv(codes, params) -> np.ndarray:
    """KV entries are decompressed without fp16 rounding (the pages use an fp32 workspace)."""
    return dequantize_exact(codes, params)


# ----------------------------------------------------------------------------- general config

def pack_bits(c: np.ndarray, num_bits: int) -> np.ndarray:
    """[..., n] codes in [0, 2^b) -> [..., n*b/8] bytes: the codes are concatenated
    least significant bit first (bit k of element i is bit b*i + k of the stream,
    stream bit t is bit t % 8 of byte t // 8).  For b = 4 this is `pack_nibbles`."""
    c = np.asarray(c, dtype=np.uint64)
    n = c.shape[-1]
    assert (n * num_bits) % 8 == 0
    bits = ((c[..., :, None] >> np.arange(num_bits, dtype=np.uint64)) & 1).astype(np.uint8)
    bits = bits.reshape(c.shape[:-1] + (n * num_bits // 8, 8))
    return (bits << np.arange(8, dtype=np.uint8)).sum(axis=-1).astype(np.uint8)


def unpack_bits(b: np.ndarray, num_bits: int) -> np.ndarray:
    """Inverse of `pack_bits`: [..., m] bytes -> [..., m*8/b] codes."""
    b = np.asarray(b, dtype=np.uint8)
    bits = ((b[..., :, None] >> np.arange(8, dtype=np.uint8)) & 1).astype(np.uint64)
    n = b.shape[-1] * 8 // num_bits
    bits = bits.reshape(b.shape[:-1] + (n, num_bits))
    return (bits << np.arange(num_bits, dtype=np.uint64)).sum(axis=-1).astype(np.uint16)


def quantize_config(x, num_bits=4, group_size=64, group_dim=-1, symmetric=False):
    """Group-wise quantization with a general CompressionConfig ([WALK] section 6.3
    names its fields num_bits, group_size, group_dim, symmetric; section 1.2 of the
    hub page mentions int3 and int4).  Readings where the pages are silent:
      * the grouped axis is zero-padded to a whole number of groups; the padding is
        quantized with its group like any element (`dequantize_config` drops it);
      * asymmetric: offset = group minimum, step = fp16(fl32(max - min) / (2^b - 1)),
        code = clamp(rne(fl32(x - min) * fl32(1 / step)), 0, 2^b - 1) -- the 4-bit
        rule with 15 replaced by 2^b - 1;
      * symmetric: B = 2^(b-1) - 1, step = fp16(fl32(max |x|) / B),
        code = clamp(rne(fl32(x) * fl32(1 / step)), -B, B), stored as code + 2^(b-1)
        (b unsigned bits), offset stored as +0;
      * a constant (asymmetric) or all-zero (symmetric) group gets step 0 and the
        code of its value; a step that underflows fp16 becomes 2^-24; a zero offset
        is stored as +0;
      * the b-bit codes of a group are packed with `pack_bits` into group_size*b/8
        bytes (group_size*b must be a multiple of 8), so the packed tensor has
        shape[:group_dim] + (num_groups * group_size * b / 8,) + shape[group_dim+1:]
        (the pages' data_shape with b = 4), and params has
        shape[:group_dim] + (num_groups,) + shape[group_dim+1:] + (2,) = (offset, step).
    Decisions are taken in fp32 in a fixed order, as in `quantize`."""
    if not 2 <= num_bits <= 8:
        raise ValueError("num_bits must be in [2, 8]")
    if group_size < 1 or (group_size * num_bits) % 8:
        raise ValueError("group_size * num_bits must be a multiple of 8")
    x = np.asarray(x, dtype=F16)
    gd = group_dim % x.ndim
    xm = np.moveaxis(x, gd, -1)
    n = xm.shape[-1]
    ng = -(-n // group_size)
    pad = ng * group_size - n
    xp = np.concatenate([xm, np.zeros(xm.shape[:-1] + (pad,), F16)], axis=-1) if pad else xm
    g = xp.reshape(xm.shape[:-1] + (ng, group_size)).astype(F32)
    if symmetric:
        qmax = (1 << (num_bits - 1)) - 1
        amax = np.abs(g).max(axis=-1)
        s = (amax / F32(qmax)).astype(F16)
        const = amax == 0
    else:
        qmax = (1 << num_bits) - 1
        mn = g.min(axis=-1)
        mx = g.max(axis=-1)
        s = ((mx - mn) / F32(qmax)).astype(F16)
        const = mx == mn
    s = np.where(const, F16(0), np.where(s == 0, F16(2.0 ** -24), s)).astype(F16)
    s32 = s.astype(F32)
    with np.errstate(divide="ignore"):
        inv = np.where(const, F32(0), F32(1) / np.where(const, F32(1), s32)).astype(F32)
    if symmetric:
        t = g * inv[..., None]
        c = np.clip(np.rint(t), -qmax, qmax).astype(np.int32) + (1 << (num_bits - 1))
        offset = np.zeros(s.shape, F16)
    else:
        t = (g - mn[..., None]) * inv[..., None]
        c = np.clip(np.rint(t), 0, qmax).astype(np.int32)
        offset = (mn + F32(0)).astype(F16)
    packed = pack_bits(c.reshape(c.shape[:-2] + (ng * group_size,)), num_bits)
    codes = np.moveaxis(packed, -1, gd)
    params = np.moveaxis(np.stack([offset, s], axis=-1).astype(F16), -2, gd)
    return codes, params


def dequantize_config(codes, params, n, num_bits=4, group_size=64, group_dim=-1,
                      symmetric=False) -> np.ndarray:
    """Exact values (float64) of `quantize_config`'s output, the grouped axis cut back
    to its n elements: code * step + offset, or (code - 2^(b-1)) * step if symmetric."""
    codes = np.asarray(codes, dtype=np.uint8)
    gd = group_dim % codes.ndim
    cm = np.moveaxis(codes, gd, -1)
    pm = np.moveaxis(np.asarray(params, dtype=F16), gd, -2)
    c = unpack_bits(cm, num_bits).astype(F64)
    ng = pm.shape[-2]
    c = c.reshape(cm.shape[:-1] + (ng, group_size))
    off = pm[..., 0].astype(F64)[..., None]
    step = pm[..., 1].astype(F64)[..., None]
    if symmetric:
        v = (c - (1 << (num_bits - 1))) * step
    else:
        v = c * step + off
    v = v.reshape(cm.shape[:-1] + (ng * group_size,))[..., :n]
    return np.moveaxis(v, -1, gd)


# ----------------------------------------------------------------------------- linear / LN

def _finish_linear(acc, bias, residual, relu, out_dtype):
    if bias is not None:
        acc = acc + np.asarray(bias, dtype=F16).astype(F64)
    if relu:
        acc = np.maximum(acc, 0.0)
    if residual is not None:
        acc = acc + np.asarray(residual, dtype=F16).astype(F64)
    return acc.astype(out_dtype)


def linear_w4(x, codes, params, bias=None, residual=None, relu=False, out_dtype=F16):
    """y = [relu](x . W^T + b) [+ residual] with W the fp16-dequantized 4-bit weight [N][K].

    One rounding to `out_dtype` at the end (fp16 for hidden states, float64 for logits).
    """
    return linear_dequantized(x, dequantize_weight(codes, params).astype(F64), bias, residual,
                              relu, out_dtype)


def linear_dequantized(x, w64, bias=None, residual=None, relu=False, out_dtype=F16):
    """`linear_w4` with the weight already dequantized (float64 copy of its fp16 values)."""
    x = np.asarray(x, dtype=F16).astype(F64)
    return _finish_linear(x @ w64.T, bias, residual, relu, out_dtype)


def linear_w4_sampled(x, codes, params, rows, cols, bias=None, residual=None, relu=False):
    """The same output as `linear_w4`, only at the (rows[i], cols[i]) positions.

    Used at sizes where the full product is out of reach on the CPU.
    """
    x = np.asarray(x, dtype=F16)
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    out = np.empty(len(rows), dtype=F16)
    for i, (m, n) in enumerate(zip(rows, cols)):
        w = dequantize_weight(codes[n], params[n]).astype(F64)
        acc = float(np.dot(x[m].astype(F64), w))
        b = None if bias is None else np.asarray(bias)[n]
        r = None if residual is None else np.asarray(residual)[m, n]
        out[i] = _finish_linear(np.array(acc), b, r, relu, F16)
    return out


def layernorm(x, gamma, beta, eps=LN_EPS) -> np.ndarray:
    """(x - mean) / sqrt(biased var + eps) * gamma + beta over the last axis, fp16 out."""
    x = np.asarray(x, dtype=F16).astype(F64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    y = (x - mu) / np.sqrt(var + eps)
    y = y * np.asarray(gamma, dtype=F16).astype(F64) + np.asarray(beta, dtype=F16).astype(F64)
    return y.astype(F16)


# ----------------------------------------------------------------------------- KV cache

class KVCache:
    """4-bit cache of one layer: codes [B][heads][max_len][hd/2], params [B][heads][max_len][hd/64][2]."""

    def __init__(self, batch, heads, head_dim, max_len):
        self.batch, self.heads, self.head_dim, self.max_len = batch, heads, head_dim, max_len
        # left padding of each cache row: positions [0, pad) hold pad tokens, never attended
        self.pad = np.zeros(batch, np.int64)
        self.k_codes = np.zeros((batch, heads, max_len, head_dim // 2), np.uint8)
        self.v_codes = np.zeros_like(self.k_codes)
        self.k_params = np.zeros((batch, heads, max_len, head_dim // GROUP, 2), F16)
        self.v_params = np.zeros_like(self.k_params)

    def store(self, b, t0, k, v):
        """Quantize fp16 k, v [heads][T][hd] into positions [t0, t0+T) of sequence b."""
        T = k.shape[1]
        self.k_codes[b, :, t0:t0 + T], self.k_params[b, :, t0:t0 + T] = quantize(k)
        self.v_codes[b, :, t0:t0 + T], self.v_params[b, :, t0:t0 + T] = quantize(v)

    def read(self, b, head, length):
        k = dequantize_kv(self.k_codes[b, head, :length], self.k_params[b, head, :length])
        v = dequantize_kv(self.v_codes[b, head, :length], self.v_params[b, head, :length])
        return k, v


def _split_qkv(qkv, heads, head_dim):
    """qkv [..., 3h] -> q, k, v [..., heads, hd]; N index = part*h + head*hd + d."""
    h = heads * head_dim
    q = qkv[..., 0:h].reshape(qkv.shape[:-1] + (heads, head_dim))
    k = qkv[..., h:2 * h].reshape(qkv.shape[:-1] + (heads, head_dim))
    v = qkv[..., 2 * h:3 * h].reshape(qkv.shape[:-1] + (heads, head_dim))
    return q, k, v


def _softmax_rows(s):
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=-1, keepdims=True)


def attn_prefill(qkv, batch, seq, heads, head_dim, cache: KVCache | None = None, b0=0, pad=None):
    """Causal attention over the prompt (the pages' `mha`), then 4-bit store of K and V.

    qkv: fp16 [batch*seq][3h], rows ordered (b, t).  Returns fp16 [batch*seq][h].
    Scores use the fp16 K/V of this pass; K and V then go to cache rows b0+b, positions [0, seq).
    Left padding (the pages' attention_mask): sequence b's first pad[b] positions (default:
    the cache rows' pad, else 0; clamped to [0, seq - 1]) are pad tokens, so query t sees
    keys pad[b] <= j <= t; a pad query sees none and its output is 0.
    """
    qkv = np.asarray(qkv, dtype=F16).reshape(batch, seq, -1)
    q, k, v = _split_qkv(qkv, heads, head_dim)         # [B][S][nh][hd]
    out = np.zeros((batch, seq, heads, head_dim), F16)
    scale = 1.0 / np.sqrt(head_dim)
    if pad is None:
        pad = cache.pad[b0:b0 + batch] if cache is not None else np.zeros(batch, np.int64)
    pad = np.clip(np.asarray(pad, np.int64), 0, seq - 1)
    causal = np.tril(np.ones((seq, seq), dtype=bool))
    for b in range(batch):
        p0 = int(pad[b])
        for hh in range(heads):
            qh = q[b, p0:, hh].astype(F64)
            kh = k[b, p0:, hh].astype(F64)
            vh = v[b, p0:, hh].astype(F64)
            s = (qh @ kh.T) * scale
            s = np.where(causal[:seq - p0, :seq - p0], s, -np.inf)
            out[b, p0:, hh] = (_softmax_rows(s) @ vh).astype(F16)
        if cache is not None:
            cache.store(b0 + b, 0, np.ascontiguousarray(k[b].transpose(1, 0, 2)),
                        np.ascontiguousarray(v[b].transpose(1, 0, 2)))
    return out.reshape(batch * seq, heads * head_dim)


def topk_count(sparsity, n):
    """Positions kept by sparse attention over n candidates: k = ceil(min(sparsity, 1) * n),
    the product taken in float32 (sparsity a float32), at least 1."""
    k = int(np.ceil(min(np.float32(sparsity), np.float32(1)) * np.float32(n)))
    return max(k, 1)


def attn_decode(qkv, pos, cache: KVCache, b0=0, sparsity=1.0):
    """One new token per sequence attends to the 4-bit cache (the pages' `mha_gen`).

    qkv: fp16 [nb][3h] for cache rows b0..b0+nb-1.  The token's k, v are quantized into
    position `pos` first; positions [pad, pos] are then read back from the 4-bit cache,
    pad = the cache row's left padding clamped to [0, pos].  Returns fp16 [nb][h].
    sparsity < 1 ([NOTES] "Flex Opt": the attn_sparsity policy): each query keeps only
    its k = topk_count(sparsity, n) highest-scoring positions of the n candidates (the
    lower position first among equal scores) and attends to them alone (softmax over
    the kept scores).
    """
    heads, head_dim = cache.heads, cache.head_dim
    qkv = np.asarray(qkv, dtype=F16)
    nb = qkv.shape[0]
    q, k, v = _split_qkv(qkv, heads, head_dim)         # [nb][nh][hd]
    out = np.empty((nb, heads, head_dim), F16)
    scale = 1.0 / np.sqrt(head_dim)
    for i in range(nb):
        cache.store(b0 + i, pos, k[i][:, None, :], v[i][:, None, :])
        p0 = int(np.clip(cache.pad[b0 + i], 0, pos))
        for hh in range(heads):
            kh, vh = cache.read(b0 + i, hh, pos + 1)
            kh, vh = kh[p0:], vh[p0:]
            s = (kh @ q[i, hh].astype(F64)) * scale
            kept = topk_count(sparsity, s.size)
            if kept < s.size:
                keep = np.lexsort((np.arange(s.size), -s))[:kept]   # by score, then position
                s, vh = s[keep], vh[keep]
            p = _softmax_rows(s[None, :])[0]
            out[i, hh] = (p @ vh).astype(F16)
    return out.reshape(nb, heads * head_dim)


# ----------------------------------------------------------------------------- OPT layer/model

class QLayer:
    """One pre-LN OPT decoder layer with 4-bit weights (codes/params per matrix)."""

    def __init__(self, w16: dict, heads: int):
        self.heads = heads
        self.hidden = w16["wo"].shape[0]
        self.head_dim = self.hidden // heads
        self.p = {k: np.asarray(v, dtype=F16) for k, v in w16.items() if not k.startswith("w")}
        self.q = {k: quantize(np.asarray(w16[k], dtype=F16)) for k in ("wqkv", "wo", "w1", "w2")}
        # weights are decompressed once (to fp16, held as float64), not on every call
        self.w = {k: dequantize_weight(*self.q[k]).astype(F64) for k in self.q}

    def _attn_block(self, x, attn_fn):
        a = layernorm(x, self.p["ln1_g"], self.p["ln1_b"])
        qkv = linear_dequantized(a, self.w["wqkv"], bias=self.p["bqkv"])
        o = attn_fn(qkv)
        return linear_dequantized(o, self.w["wo"], bias=self.p["bo"], residual=x)

    def _mlp_block(self, x1):
        a = layernorm(x1, self.p["ln2_g"], self.p["ln2_b"])
        u = linear_dequantized(a, self.w["w1"], bias=self.p["b1"], relu=True)
        return linear_dequantized(u, self.w["w2"], bias=self.p["b2"], residual=x1)

    def prefill(self, x, batch, seq, cache, b0=0):
        """x fp16 [batch*seq][h] -> fp16 [batch*seq][h]; fills cache positions [0, seq)."""
        x1 = self._attn_block(x, lambda qkv: attn_prefill(qkv, batch, seq, self.heads,
                                                          self.head_dim, cache, b0))
        return self._mlp_block(x1)

    def decode(self, x, pos, cache, b0=0, sparsity=1.0):
        """x fp16 [nb][h] (one token per sequence at position pos) -> fp16 [nb][h]."""
        x1 = self._attn_block(x, lambda qkv: attn_decode(qkv, pos, cache, b0, sparsity))
        return self._mlp_block(x1)


def embed(tokens, positions, e_codes, e_params, pos_table, pos_offset=2):
    """fp16(dequantized token row + learned position row at position + offset) (`opt_input_embed`)."""
    tokens = np.asarray(tokens).reshape(-1)
    positions = np.asarray(positions).reshape(-1)
    tok = dequantize_weight(e_codes[tokens], e_params[tokens]).astype(F64)
    pos = np.asarray(pos_table, dtype=F16)[positions + pos_offset].astype(F64)
    return (tok + pos).astype(F16)


def lm_head(x_last, lnf_g, lnf_b, e_codes, e_params, e_w64=None):
    """Final LayerNorm, logits against the tied 4-bit embedding (no bias), greedy pick.

    Returns (logits float64 [nb][V], next token int32 [nb]); np.argmax takes the lowest
    index among equal maxima.  e_w64: the embedding already dequantized, if at hand.
    """
    a = layernorm(x_last, lnf_g, lnf_b)
    if e_w64 is None:
        e_w64 = dequantize_weight(e_codes, e_params).astype(F64)
    logits = linear_dequantized(a, e_w64, out_dtype=F64)
    return logits, np.argmax(logits, axis=-1).astype(np.int32)


# ----------------------------------------------------------------------------- sampling

GOLDEN64 = 0x9E3779B97F4A7C15


def splitmix64(seed: int, counter) -> np.ndarray:
    """Output number `counter` (0, 1, ...) of the SplitMix64 generator started from
    state `seed`: mix(seed + (counter + 1) * golden) with the published constants
    (0x9E3779B97F4A7C15; multipliers 0xBF58476D1CE4E5B9, 0x94D049BB133111EB; shifts 30,
    27, 31), arithmetic mod 2^64 -- a counter-based generator."""
    c = np.asarray(counter, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + (c + np.uint64(1)) * np.uint64(GOLDEN64)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def sample_uniform(seed: int, step: int, rows, n: int) -> np.ndarray:
    """Uniform draws in (0, 1), one per (sequence, token) of generation step `step`:
    counter = step * 2^48 + sequence * 2^32 + token, u = ((z >> 12) + 1/2) * 2^-52,
    the top 52 bits of the output centred in their cell (exact in float64, so u lies in
    [2^-53, 1 - 2^-53])."""
    rows = np.asarray(rows, dtype=np.uint64)[:, None]
    tok = np.arange(n, dtype=np.uint64)[None, :]
    counter = (np.uint64(step) << np.uint64(48)) | (rows << np.uint64(32)) | tok
    z = splitmix64(seed, counter)
    return ((z >> np.uint64(12)).astype(F64) + 0.5) * 2.0 ** -52


def pick(logits, gen=None, step=0, m0=0, stopped=None):
    """Next tokens from fp32 logits [M][N] ([WALK] section 4.1: `generate(input_ids,
    do_sample, temperature, max_new_tokens, stop)`).  Readings where the pages are
    silent:
      * do_sample=False: greedy, the lowest index among equal maxima;
      * do_sample=True: a draw from softmax(logits / temperature) by the Gumbel-max
        rule: argmax_n (logit_n / T + g_n), g_n = -log(-log u_n) with the counter-based
        uniforms of `sample_uniform` (sequence m0 + m, step = the position of the
        token the logits follow), in float64, lowest index among equal maxima;
      * stop (a token id, or -1 for none): a sequence that has produced it is stopped
        and keeps producing it; `stopped` (bool [M], updated in place) carries that
        across steps.
    `gen` is None or a dict with do_sample, temperature, seed, stop."""
    lg = np.asarray(logits, dtype=np.float32)
    M, N = lg.shape
    if gen is not None and gen.get("do_sample"):
        u = sample_uniform(gen["seed"], step, np.arange(m0, m0 + M), N)
        score = lg.astype(F64) / F64(np.float32(gen["temperature"])) - np.log(-np.log(u))
        nxt = score.argmax(axis=1)
    else:
        nxt = lg.argmax(axis=1)
    nxt = nxt.astype(np.int64)
    stop = -1 if gen is None else int(gen.get("stop", -1))
    if stopped is not None and stop >= 0:
        nxt = np.where(stopped, stop, nxt)
        stopped |= nxt == stop
    return nxt


class QModel:
    """OPT-shaped model: embedding, N decoder layers, output head ([NOTES] "Flex Opt")."""

    def __init__(self, layers: list, embed16, pos16, lnf_g, lnf_b, heads: int):
        self.layers = layers
        self.heads = heads
        self.e_codes, self.e_params = quantize(np.asarray(embed16, dtype=F16))
        self.e_w = dequantize_weight(self.e_codes, self.e_params).astype(F64)
        self.pos = np.asarray(pos16, dtype=F16)
        self.lnf_g = np.asarray(lnf_g, dtype=F16)
        self.lnf_b = np.asarray(lnf_b, dtype=F16)

    def new_caches(self, batch, max_len):
        return [KVCache(batch, L.heads, L.head_dim, max_len) for L in self.layers]

    def prefill(self, tokens, caches, b0=0, pad=None):
        """tokens int [nb][S] -> (logits [nb][V], next token [nb]).

        pad: left padding of each sequence (default 0; clamped to [0, S - 1]), recorded in
        the caches' rows b0.. for the decode steps.  A token's position counts from its
        sequence's first real token (pad tokens take position 0)."""
        tokens = np.asarray(tokens)
        nb, seq = tokens.shape
        pad = np.zeros(nb, np.int64) if pad is None else np.clip(np.asarray(pad, np.int64), 0,
                                                                     seq - 1)
        for c in caches:
            c.pad[b0:b0 + nb] = pad
        positions = np.maximum(np.arange(seq)[None, :] - pad[:, None], 0).reshape(-1)
        x = embed(tokens, positions, self.e_codes, self.e_params, self.pos)
        for L, c in zip(self.layers, caches):
            x = L.prefill(x, nb, seq, c, b0)
        last = x.reshape(nb, seq, -1)[:, -1]
        return lm_head(last, self.lnf_g, self.lnf_b, self.e_codes, self.e_params, self.e_w)

    def decode_step(self, tokens, pos, caches, b0=0, sparsity=1.0):
        """tokens int [nb] at position pos -> (logits [nb][V], next token [nb])."""
        tokens = np.asarray(tokens).reshape(-1)
        positions = np.maximum(pos - caches[0].pad[b0:b0 + tokens.size], 0)
        x = embed(tokens, positions, self.e_codes, self.e_params, self.pos)
        for L, c in zip(self.layers, caches):
            x = L.decode(x, pos, c, b0, sparsity)
        return lm_head(x, self.lnf_g, self.lnf_b, self.e_codes, self.e_params, self.e_w)

    def generate(self, tokens, gen, config=None, pad=None, sparsity=1.0):
        """Generation of `gen` tokens ([WALK] section 4.1): greedy without `config`, else
        `pick` with it (do_sample, temperature, seed, stop); `pad` = left padding of each
        prompt (the attention mask of a ragged batch); `sparsity` < 1: top-k decode
        attention (see attn_decode)."""
        tokens = np.asarray(tokens)
        nb, seq = tokens.shape
        caches = self.new_caches(nb, seq + gen - 1)
        stopped = np.zeros(nb, dtype=bool)
        lg, nxt = self.prefill(tokens, caches, pad=pad)
        if config is not None:
            nxt = pick(lg, config, seq - 1, 0, stopped)
        out = [nxt]
        for i in range(gen - 1):
            lg, nxt = self.decode_step(nxt, seq + i, caches, sparsity=sparsity)
            if config is not None:
                nxt = pick(lg, config, seq + i, 0, stopped)
            out.append(nxt)
        return np.stack(out, axis=1)
