"""Kernel-level parity of the HIP library against the oracle (needs an MI355X).

Both sides receive the same fp16 bytes.  Integer outputs (codes, offsets, scales,
argmax) must match bit for bit; floating outputs within a bound derived from fp32
accumulation (GPU) versus float64 (oracle) plus one fp16 rounding.
"""
import numpy as np
import pytest
import torch

from oracle import flexq_oracle as O
from tests.gpu_helpers import F16, assert_close_fp16, require_gpu, to_np

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _groups_mix(rng, rows, cols):
    x = rng.normal(size=(rows, cols))
    g = x.reshape(rows, cols // 64, 64)
    n = g.shape[1]
    sel = rng.random((rows, n))
    g[sel < 0.05] = 3.25                                          # constant groups
    g[(sel >= 0.05) & (sel < 0.08)] = 0.0                         # zero groups
    tiny = (sel >= 0.08) & (sel < 0.10)
    g[tiny] = rng.integers(0, 3, size=(tiny.sum(), 64)) * 2.0**-24  # step underflows
    scale = 8.0 ** rng.integers(-6, 4, size=(rows, n, 1))
    g *= np.where(((sel >= 0.10) & (sel < 0.4))[..., None], scale, 1.0)
    out = rng.random(g.shape) < 0.01
    g[out] *= 8
    ties = (sel >= 0.4) & (sel < 0.45)           # step exactly 1, values on k + 1/2
    k = rng.integers(0, 15, size=(ties.sum(), 64)) + 0.5
    k[:, 0], k[:, 1] = 0.0, 15.0
    g[ties] = k + rng.choice([0.0, -8.0, 32.0], size=(ties.sum(), 1))
    x = g.reshape(rows, cols).astype(F16)
    negz = rng.random(x.shape) < 0.02
    x[negz & (x == 0)] = F16(-0.0)
    assert np.isfinite(x).all()
    return x


@pytest.mark.parametrize("rows,cols", [(1, 64), (37, 768), (256, 4096), (3, 12288)])
def test_quantize_bit_exact(rows, cols):
    F = require_gpu()
    _say("quantize", rows, cols)
    rng = np.random.default_rng(rows * 131 + cols)
    x = _groups_mix(rng, rows, cols)
    w = F.quantize(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    codes, params = O.quantize(x)
    assert np.array_equal(to_np(w.codes), codes)
    assert np.array_equal(to_np(w.params).view(np.uint16), params.view(np.uint16))


@pytest.mark.parametrize("rows,cols", [(1, 64), (200, 768), (384, 128), (3, 12288)])
def test_quantize_weight_layout_bit_exact(rows, cols):
    """flexq_quantize_w4: the oracle's codes and params, placed where flexq_w4 says
    (checked through the documented byte/word formulas), pad rows zero."""
    F = require_gpu()
    _say("quantize_w4", rows, cols)
    rng = np.random.default_rng(rows * 17 + cols)
    x = _groups_mix(rng, rows, cols)
    w = F.quantize_weight(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    codes, params = O.quantize(x)
    flat_c = to_np(w.codes).reshape(-1)
    flat_p = to_np(w.params).view(np.uint32).reshape(-1)
    KT = cols // 64
    r = np.arange(rows)[:, None]
    kt = np.arange(KT)[None, :]
    base = ((r // 128) * KT + kt) * 4096 + (r % 128) * 32
    got_c = flat_c[base[:, :, None] + np.arange(32)[None, None, :]].reshape(rows, KT, 8, 4)
    # byte 4 q + j of a k-tile holds elements 8 q + j (low nibble) and 8 q + j + 4 (high)
    el = np.concatenate((got_c & 15, got_c >> 4), axis=-1).reshape(rows, cols)
    assert np.array_equal(el, O.unpack_nibbles(codes))
    got_p = flat_p[((r // 128) * KT + kt) * 128 + (r % 128)]
    assert np.array_equal(got_p, params.view(np.uint32).reshape(rows, KT))
    nb = (rows + 127) // 128
    assert flat_c.size == nb * 128 * cols // 2
    pad = np.ones((nb * 128, KT), bool)
    pad[:rows] = False
    prow = np.nonzero(pad[:, 0])[0]
    if prow.size:
        pb = ((prow[:, None] // 128) * KT + kt) * 4096 + (prow[:, None] % 128) * 32
        assert not flat_c[pb[:, :, None] + np.arange(32)].any()
        assert not flat_p[((prow[:, None] // 128) * KT + kt) * 128 + prow[:, None] % 128].any()
    c2, p2 = w.rowmajor()
    assert np.array_equal(to_np(c2), codes)


def test_quantize_rejects_bad_config():
    F = require_gpu()
    import ctypes as C
    x = torch.zeros(4, 64, dtype=torch.float16, device="cuda")
    w = F.Q4.empty(4, 64)
    L = F.lib()
    st = L.flexq_quantize(x.data_ptr(), 4, 64, F.QConfig(3, 64, 0), w.codes.data_ptr(),
                          w.params.data_ptr(), C.c_void_p(0))
    assert st == F.ERR_UNSUPPORTED
    st = L.flexq_quantize(x.data_ptr(), 4, 96, F.QConfig(4, 64, 0), w.codes.data_ptr(),
                          w.params.data_ptr(), C.c_void_p(0))
    assert st == F.ERR_INVALID


def test_dequantize_bit_exact():
    F = require_gpu()
    _say("dequantize")
    rng = np.random.default_rng(7)
    rows, cols = 512, 1024
    codes = rng.integers(0, 256, size=(rows, cols // 2)).astype(np.uint8)
    # scales/offsets across the fp16 range, subnormals included
    s = (np.abs(rng.normal(size=(rows, cols // 64))) * 2.0 ** rng.integers(-26, 10, size=(rows, cols // 64))).astype(F16)
    m = (rng.normal(size=(rows, cols // 64)) * 2.0 ** rng.integers(-20, 12, size=(rows, cols // 64))).astype(F16)
    params = np.stack([m, s], axis=-1).astype(F16)
    w = F.Q4(torch.from_numpy(codes).cuda(), torch.from_numpy(params).cuda())
    got = to_np(F.dequantize(w))
    ref = O.dequantize_weight(codes, params)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))


def _bound_linear(x, w16, K):
    """fp32-accumulation error bound: K * 2^-24 * sum|x||w| (plus the final fp16 ulp)."""
    return K * 2.0**-24 * (np.abs(x.astype(np.float64)) @ np.abs(w16.astype(np.float64)).T)


@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (5, 200, 320), (32, 384, 1024), (37, 128, 256),
                                   (64, 256, 512), (80, 1152, 384), (129, 1000, 1024), (144, 384, 768),
                                   (100, 200, 64), (144, 64, 4096),
                                   (144, 33792, 4096), (97, 33792, 2048),   # decode kernel, two splits
                                   (160, 128, 128),
                                   (300, 256, 640), (513, 192, 1024), (4, 256, 8192),
                                   # k-loop remainders: large-M kernel with an odd k-tile
                                   # count (9; 45 in 5 splits of 9), small-M kernel with 7,
                                   # decode kernel with 4 and 3 left after its 5-stage
                                   # groups (M x N not a multiple of 4 keeps K unsplit)
                                   (400, 320, 576), (300, 256, 2880), (41, 250, 448),
                                   (143, 382, 576), (121, 254, 512),
                                   # decode kernel with 6 row tiles of 16 (81 <= M <= 96)
                                   (90, 384, 512)])
@pytest.mark.parametrize("epi", ["plain", "bias_relu", "bias_res"])
def test_linear_w4(M, N, K, epi):
    F = require_gpu()
    _say("linear", M, N, K, epi)
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    x = rng.normal(size=(M, K)).astype(F16)
    w = (rng.normal(size=(N, K)) * 0.05).astype(F16)
    bias = (rng.normal(size=N) * 0.5).astype(F16) if epi != "plain" else None
    res = rng.normal(size=(M, N)).astype(F16) if epi == "bias_res" else None
    relu = epi == "bias_relu"
    codes, params = O.quantize(w)
    wq = F.W4.from_rowmajor(torch.from_numpy(codes).cuda(), torch.from_numpy(params).cuda())
    y = F.linear_w4(torch.from_numpy(x).cuda(), wq,
                    bias=None if bias is None else torch.from_numpy(bias).cuda(),
                    residual=None if res is None else torch.from_numpy(res).cuda(), relu=relu)
    got = to_np(y)
    ref = O.linear_w4(x, codes, params, bias=bias, residual=res, relu=relu)
    wd = O.dequantize_weight(codes, params)
    assert_close_fp16(got, ref, extra=_bound_linear(x, wd, K) + 1e-7, what=f"linear {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(3, 50272 // 8, 768), (144, 1000, 512), (2, 96, 4096),
                                   # large-M kernel writing fp32, direct and split-K
                                   (300, 200, 640), (300, 256, 2048)])
def test_linear_w4_f32(M, N, K):
    F = require_gpu()
    _say("linear_f32", M, N, K)
    rng = np.random.default_rng(N + K)
    x = rng.normal(size=(M, K)).astype(F16)
    w = (rng.normal(size=(N, K)) * 0.05).astype(F16)
    codes, params = O.quantize(w)
    wq = F.W4.from_rowmajor(torch.from_numpy(codes).cuda(), torch.from_numpy(params).cuda())
    got = to_np(F.linear_w4_f32(torch.from_numpy(x).cuda(), wq)).astype(np.float64)
    ref = O.linear_w4(x, codes, params, out_dtype=np.float64)
    wd = O.dequantize_weight(codes, params)
    bound = _bound_linear(x, wd, K) + np.abs(ref) * 2.0**-23
    assert np.all(np.abs(got - ref) <= bound)


def test_linear_in_place_residual():
    F = require_gpu()
    rng = np.random.default_rng(3)
    M, N, K = 48, 256, 256
    x = rng.normal(size=(M, K)).astype(F16)
    w = (rng.normal(size=(N, K)) * 0.05).astype(F16)
    r = rng.normal(size=(M, N)).astype(F16)
    codes, params = O.quantize(w)
    wq = F.W4.from_rowmajor(torch.from_numpy(codes).cuda(), torch.from_numpy(params).cuda())
    rt = torch.from_numpy(r).cuda()
    F.linear_w4(torch.from_numpy(x).cuda(), wq, residual=rt, out=rt)
    ref = O.linear_w4(x, codes, params, residual=r)
    assert_close_fp16(to_np(rt), ref, extra=_bound_linear(x, O.dequantize_weight(codes, params), K))


@pytest.mark.parametrize("M,h,stride", [(1, 128, 128), (33, 768, 768), (5, 12288, 12288),
                                        (4, 2048, 3 * 2048)])
def test_layernorm(M, h, stride):
    F = require_gpu()
    _say("layernorm", M, h, stride)
    rng = np.random.default_rng(h + M)
    xs = (rng.normal(size=(M, stride)) * 3 + 1).astype(F16)
    g = (1 + rng.normal(size=h) * 0.1).astype(F16)
    b = (rng.normal(size=h) * 0.1).astype(F16)
    y = F.layernorm(torch.from_numpy(xs).cuda(), torch.from_numpy(g).cuda(), torch.from_numpy(b).cuda(),
                    rows=M, row_stride=stride)
    ref = O.layernorm(xs[:, :h], g, b)
    # fp32 statistics: a few ulp of the normalised value times |g|, plus one fp16 rounding
    extra = 1e-5 * (np.abs(ref.astype(np.float64)) + 1) * np.abs(g.astype(np.float64)) * 8
    assert_close_fp16(to_np(y), ref, extra=extra, what="layernorm")


def _make_qkv(rng, B, S, nh, hd):
    return rng.normal(size=(B * S, 3 * nh * hd)).astype(F16)


@pytest.mark.parametrize("B,S,nh,hd", [(1, 1, 1, 64), (2, 17, 3, 64), (2, 130, 2, 128),
                                       (1, 64, 4, 128), (3, 200, 2, 64), (2, 300, 2, 128),
                                       (1, 512, 3, 128), (2, 385, 2, 64)])
def test_attn_prefill(B, S, nh, hd):
    F = require_gpu()
    _say("attn_prefill", B, S, nh, hd)
    rng = np.random.default_rng(B * 1000 + S * 10 + hd)
    qkv = _make_qkv(rng, B, S, nh, hd)
    b0 = 1
    kv = F.KV4(B + 2, nh, hd, S + 5)
    out = F.attn_prefill(torch.from_numpy(qkv).cuda(), B, S, kv, b0=b0)
    torch.cuda.synchronize()
    oc = O.KVCache(B + 2, nh, hd, S + 5)
    ref = O.attn_prefill(qkv, B, S, nh, hd, oc, b0=b0)
    # fp16 probabilities feed the P.V product: relative 2^-11 per weight, plus fp32 sums
    vmax = np.abs(qkv.astype(np.float64)).max()
    assert_close_fp16(to_np(out), ref, extra=2.0**-10 * vmax, what="prefill out")
    for name in ("k_codes", "v_codes"):
        assert np.array_equal(to_np(getattr(kv, name)), getattr(oc, name)), name
    for name in ("k_params", "v_params"):
        assert np.array_equal(to_np(getattr(kv, name)).view(np.uint16),
                              getattr(oc, name).view(np.uint16)), name


@pytest.mark.parametrize("B,nh,hd,S,steps", [(2, 3, 64, 5, 4), (4, 12, 64, 128, 3),
                                             (1, 2, 128, 700, 3), (3, 2, 128, 64, 70)])
def test_attn_decode(B, nh, hd, S, steps):
    F = require_gpu()
    _say("attn_decode", B, nh, hd, S, steps)
    rng = np.random.default_rng(B * 100 + S + hd)
    T = S + steps
    kv = F.KV4(B, nh, hd, T)
    oc = O.KVCache(B, nh, hd, T)
    qkv = _make_qkv(rng, B, S, nh, hd)
    F.attn_prefill(torch.from_numpy(qkv).cuda(), B, S, kv)
    O.attn_prefill(qkv, B, S, nh, hd, oc)
    for i in range(steps):
        pos = S + i
        q1 = rng.normal(size=(B, 3 * nh * hd)).astype(F16)
        out = F.attn_decode(torch.from_numpy(q1).cuda(), pos, kv)
        torch.cuda.synchronize()
        ref = O.attn_decode(q1, pos, oc)
        vmax = 15 * np.abs(oc.v_params[..., 1].astype(np.float64)).max() + \
            np.abs(oc.v_params[..., 0].astype(np.float64)).max()
        assert_close_fp16(to_np(out), ref, extra=2.0**-16 * vmax, what=f"decode pos {pos}")
        assert np.array_equal(to_np(kv.k_codes), oc.k_codes)
        assert np.array_equal(to_np(kv.v_codes), oc.v_codes)
        assert np.array_equal(to_np(kv.k_params).view(np.uint16), oc.k_params.view(np.uint16))


def test_embed_and_argmax():
    F = require_gpu()
    _say("embed/argmax")
    rng = np.random.default_rng(11)
    V, h = 1000, 256
    e16 = (rng.normal(size=(V, h)) * 0.5).astype(F16)
    pos = rng.normal(size=(40, h)).astype(F16)
    codes, params = O.quantize(e16)
    ew = F.W4.from_rowmajor(torch.from_numpy(codes).cuda(), torch.from_numpy(params).cuda())
    toks = rng.integers(0, V, size=12).astype(np.int32)
    got = to_np(F.embed(torch.from_numpy(toks).cuda(), 3, 4, ew, torch.from_numpy(pos).cuda()))
    ref = O.embed(toks, 3 + np.arange(12) % 4, codes, params, pos)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
    lg = rng.normal(size=(7, 50272)).astype(np.float32)
    lg[3, 100] = lg[3, 20000] = 50.0          # tie -> lowest index
    nxt = to_np(F.argmax(torch.from_numpy(lg).cuda()))
    assert np.array_equal(nxt, lg.argmax(1))
    assert nxt[3] == 100
