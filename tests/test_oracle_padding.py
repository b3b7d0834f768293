"""Pins of the oracle's ragged (left-padded) prompts against their defining property: a
padded sequence computes exactly what the same tokens compute alone, unpadded, in every
op (prefill attention, the 4-bit cache rows, decode attention) and in whole greedy
generation; pad tokens' ids never matter; a pad query's attention output is 0."""
import numpy as np
import pytest

from oracle import flexq_oracle as O
from tests.test_oracle_model import _tiny_model

F16 = np.float16


def _qkv(rng, rows, heads, hd):
    return (rng.normal(size=(rows, 3 * heads * hd))).astype(F16)


@pytest.mark.parametrize("pad", [0, 1, 5, 9])
def test_prefill_attention_padded_equals_unpadded(pad, rng):
    S, nh, hd = 10, 2, 64
    qkv = _qkv(rng, S, nh, hd)
    c1 = O.KVCache(1, nh, hd, S)
    out = O.attn_prefill(qkv, 1, S, nh, hd, c1, pad=[pad])
    c2 = O.KVCache(1, nh, hd, S)
    ref = O.attn_prefill(qkv[pad:], 1, S - pad, nh, hd, c2)
    assert np.array_equal(out[pad:], ref)
    assert not out[:pad].any()
    assert np.array_equal(c1.k_codes[:, :, pad:], c2.k_codes[:, :, :S - pad])
    assert np.array_equal(c1.v_params[:, :, pad:], c2.v_params[:, :, :S - pad])


def test_prefill_attention_reads_pad_from_cache_rows(rng):
    S, nh, hd = 8, 1, 64
    qkv = _qkv(rng, 2 * S, nh, hd)
    c = O.KVCache(4, nh, hd, S)
    c.pad[:] = [0, 0, 3, 6]
    a = O.attn_prefill(qkv, 2, S, nh, hd, c, b0=2)
    b = O.attn_prefill(qkv, 2, S, nh, hd, None, pad=[3, 6])
    assert np.array_equal(a, b)


@pytest.mark.parametrize("pad", [0, 3, 7])
def test_decode_attention_padded_equals_unpadded(pad, rng):
    S, nh, hd, G = 8, 2, 128, 3
    c1 = O.KVCache(1, nh, hd, S + G)
    c2 = O.KVCache(1, nh, hd, S + G)
    pre = _qkv(rng, S, nh, hd)
    O.attn_prefill(pre, 1, S, nh, hd, c1, pad=[pad])
    c1.pad[0] = pad
    O.attn_prefill(pre[pad:], 1, S - pad, nh, hd, c2)
    for i in range(G):
        x = _qkv(rng, 1, nh, hd)
        a = O.attn_decode(x, S + i, c1)
        b = O.attn_decode(x, S - pad + i, c2)
        assert np.array_equal(a, b)


def test_ragged_generation_equals_each_sequence_alone(rng):
    m = _tiny_model(rng, L=2, h=128, nh=2, f=256, V=300)
    lens = [9, 4, 1]
    S, G = max(lens), 5
    toks = rng.integers(0, 300, size=(3, S))
    pad = np.array([S - n for n in lens])
    caches = m.new_caches(3, S + G - 1)
    lg, nxt = m.prefill(toks, caches, pad=pad)
    logits, out = [lg], [nxt]
    for i in range(G - 1):
        lg, nxt = m.decode_step(nxt, S + i, caches)
        logits.append(lg)
        out.append(nxt)
    out = np.stack(out, 1)
    assert np.array_equal(out, m.generate(toks, G, pad=pad))
    for b, n in enumerate(lens):
        c1 = m.new_caches(1, n + G - 1)
        lg1, nx1 = m.prefill(toks[b:b + 1, S - n:], c1)
        assert np.array_equal(nx1, out[b:b + 1, 0])
        np.testing.assert_allclose(lg1[0], logits[0][b], rtol=0, atol=1e-12)
        for i in range(G - 1):
            lg1, nx1 = m.decode_step(out[b:b + 1, i], n + i, c1)
            assert nx1[0] == out[b, i + 1]
            np.testing.assert_allclose(lg1[0], logits[i + 1][b], rtol=0, atol=1e-12)


def test_pad_token_ids_do_not_matter(rng):
    m = _tiny_model(rng, L=1, h=128, nh=2, f=256, V=300)
    S = 7
    toks = rng.integers(0, 300, size=(2, S))
    pad = np.array([4, 2])
    other = toks.copy()
    other[0, :4] = rng.integers(0, 300, size=4)
    other[1, :2] = 0
    la, _ = m.prefill(toks, m.new_caches(2, S), pad=pad)
    lb, _ = m.prefill(other, m.new_caches(2, S), pad=pad)
    assert np.array_equal(la, lb)
