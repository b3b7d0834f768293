"""Pins for the oracle's prefill attention (mha) and 4-bit-KV decode attention (mha_gen)."""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import flexq_oracle as O
from tests.oracle_helpers import F16, grid_matrix


def _qkv(rng, B, S, nh, hd, scale=1.0):
    return (rng.normal(size=(B * S, 3 * nh * hd)) * scale).astype(F16)


def _parts(qkv, B, S, nh, hd):
    h = nh * hd
    x = qkv.reshape(B, S, 3, nh, hd)
    return x[:, :, 0], x[:, :, 1], x[:, :, 2]          # [B][S][nh][hd]


def test_prefill_single_token_returns_v(rng):
    B, S, nh, hd = 2, 1, 3, 64
    qkv = _qkv(rng, B, S, nh, hd)
    out = O.attn_prefill(qkv, B, S, nh, hd)
    _, _, v = _parts(qkv, B, S, nh, hd)
    assert np.array_equal(out, v.reshape(B * S, nh * hd))


@pytest.mark.parametrize("zero_q", [False, True])
def test_prefill_equal_scores_give_causal_prefix_mean(rng, zero_q):
    # identical keys (or q = 0): every allowed score ties -> row i is the mean of v_0..v_i
    B, S, nh, hd = 2, 9, 2, 64
    qkv = _qkv(rng, B, S, nh, hd)
    x = qkv.reshape(B, S, 3, nh, hd)
    if zero_q:
        x[:, :, 0] = 0
    else:
        x[:, :, 1] = x[:, :1, 1]
    qkv = x.reshape(B * S, -1)
    out = O.attn_prefill(qkv, B, S, nh, hd).reshape(B, S, nh, hd).astype(np.float64)
    v = x[:, :, 2].astype(np.float64)
    want = np.cumsum(v, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    # one fp16 rounding of the exact mean: at most half an fp16 ulp (plus float64 noise)
    half_ulp = 0.5 * np.spacing(np.abs(want).astype(F16)).astype(np.float64)
    assert np.all(np.abs(out - want) <= half_ulp * (1 + 1e-9) + 1e-15)


def test_prefill_dominant_key_selects_its_value(rng):
    B, S, nh, hd = 1, 6, 1, 64
    x = np.zeros((B, S, 3, nh, hd))
    x[0, :, 0, 0, 0] = 30.0               # q along e0
    x[0, 0, 1, 0, 0] = 30.0               # only key 0 aligns: score 900/8 above the rest
    x[0, :, 2] = rng.normal(size=(S, nh, hd))
    qkv = x.reshape(B * S, -1).astype(F16)
    out = O.attn_prefill(qkv, B, S, nh, hd).astype(np.float64)
    v0 = qkv.reshape(B, S, 3, nh, hd)[0, 0, 2].reshape(-1).astype(np.float64)
    assert np.allclose(out, v0[None, :], atol=1e-3)


def test_prefill_matches_library_softmax(rng):
    B, S, nh, hd = 2, 7, 2, 128
    qkv = _qkv(rng, B, S, nh, hd)
    out = O.attn_prefill(qkv, B, S, nh, hd).reshape(B, S, nh, hd).astype(np.float64)
    q, k, v = (t.astype(np.float64) for t in _parts(qkv, B, S, nh, hd))
    for b in range(B):
        for hh in range(nh):
            for i in range(S):
                p = softmax(k[b, :i + 1, hh] @ q[b, i, hh] / np.sqrt(hd))
                ref = (p @ v[b, :i + 1, hh]).astype(F16).astype(np.float64)
                d = np.abs(out[b, i, hh] - ref)
                assert np.all(d <= np.abs(np.spacing(ref.astype(np.float32))) * 8192), (b, hh, i)


def test_prefill_stores_quantized_kv(rng):
    B, S, nh, hd = 2, 5, 2, 128
    qkv = _qkv(rng, B, S, nh, hd)
    cache = O.KVCache(B + 1, nh, hd, S + 3)
    O.attn_prefill(qkv, B, S, nh, hd, cache, b0=1)
    _, k, v = _parts(qkv, B, S, nh, hd)
    for b in range(B):
        for hh in range(nh):
            kc, kp = O.quantize(k[b, :, hh])
            vc, vp = O.quantize(v[b, :, hh])
            assert np.array_equal(cache.k_codes[b + 1, hh, :S], kc)
            assert np.array_equal(cache.k_params[b + 1, hh, :S], kp)
            assert np.array_equal(cache.v_codes[b + 1, hh, :S], vc)
            assert np.array_equal(cache.v_params[b + 1, hh, :S], vp)
    assert not cache.k_codes[0].any() and not cache.k_codes[:, :, S:].any()


def test_decode_first_position_returns_dequantized_v(rng):
    B, nh, hd = 3, 2, 64
    qkv = _qkv(rng, B, 1, nh, hd)
    cache = O.KVCache(B, nh, hd, 4)
    out = O.attn_decode(qkv, 0, cache)
    v = qkv[:, 2 * nh * hd:].reshape(B, nh, hd)
    vh = O.dequantize_kv(*O.quantize(v))
    assert np.array_equal(out.reshape(B, nh, hd), vh.astype(F16))
    kc, kp = O.quantize(qkv[:, nh * hd:2 * nh * hd].reshape(B, nh, hd))
    assert np.array_equal(cache.k_codes[:, :, 0], kc) and np.array_equal(cache.k_params[:, :, 0], kp)


def test_decode_equals_prefill_on_exactly_representable_kv(rng):
    # K/V rows that the 4-bit code represents exactly: decode at position t over the
    # cache must reproduce row t of prefill attention over the fp16 K/V
    B, S, nh, hd = 2, 11, 2, 128
    qkv = _qkv(rng, B, S, nh, hd).reshape(B, S, 3, nh, hd)
    kv = grid_matrix(rng, B * S * 2 * nh, hd, emin=-5, emax=-3)[0]
    qkv[:, :, 1:] = kv.reshape(B, S, 2, nh, hd)
    flat = qkv.reshape(B * S, -1)
    ref = O.attn_prefill(flat, B, S, nh, hd).reshape(B, S, -1)
    cache = O.KVCache(B, nh, hd, S)
    for t in range(S):
        out = O.attn_decode(qkv[:, t].reshape(B, -1), t, cache)
        d = np.abs(out.astype(np.float64) - ref[:, t].astype(np.float64))
        assert np.all(d <= np.abs(np.spacing(ref[:, t].astype(np.float32))) * 8192), t


def test_decode_is_independent_per_sequence(rng):
    B, nh, hd, T = 3, 2, 64, 6
    cache = O.KVCache(B, nh, hd, T)
    solo = O.KVCache(1, nh, hd, T)
    for t in range(T):
        qkv = _qkv(rng, B, 1, nh, hd)
        both = O.attn_decode(qkv, t, cache)
        one = O.attn_decode(qkv[2:3], t, solo)
        assert np.array_equal(both[2:3], one)
