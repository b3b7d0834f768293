"""Pins of the oracle's sparse decode attention (`attn_decode(..., sparsity)`): the kept
count, the one-position limit (output = that position's value), the kept set against a
brute-force search over all k-subsets (the top-k set is the one with the largest score
sum), the lower-position-first rule on equal scores, the dense limit, and padding (only
real positions compete)."""
import itertools

import numpy as np
import pytest

from oracle import flexq_oracle as O

F16 = np.float16


def test_topk_count():
    assert O.topk_count(0.25, 10) == 3          # ceil(2.5)
    assert O.topk_count(0.3, 10) == 3           # float32(0.3) * 10 rounds to 3 in float32
    assert O.topk_count(0.7, 10) == 7
    assert O.topk_count(1.0, 529) == 529
    assert O.topk_count(2.0, 5) == 5
    assert O.topk_count(1e-6, 100) == 1
    assert O.topk_count(0.5, 1) == 1


def _cache(rng, nh, hd, T, filled):
    c = O.KVCache(1, nh, hd, T)
    k = rng.normal(size=(nh, filled, hd)).astype(F16)
    v = rng.normal(size=(nh, filled, hd)).astype(F16)
    c.store(0, 0, k, v)
    return c


def _scores(c, q, pos, hh):
    kh, _ = c.read(0, hh, pos + 1)
    return (kh @ q.astype(np.float64)) / np.sqrt(c.head_dim)


def test_single_position_returns_its_value(rng):
    nh, hd, S = 2, 64, 30
    c = _cache(rng, nh, hd, S + 1, S)
    qkv = rng.normal(size=(1, 3 * nh * hd)).astype(F16)
    out = O.attn_decode(qkv, S, c, sparsity=1e-6)
    q = qkv[0, :nh * hd].reshape(nh, hd)
    for hh in range(nh):
        s = _scores(c, q[hh], S, hh)
        _, vh = c.read(0, hh, S + 1)
        assert np.array_equal(out[0, hh * hd:(hh + 1) * hd], vh[int(np.argmax(s))].astype(F16))


@pytest.mark.parametrize("n,k", [(6, 2), (7, 3), (8, 5)])
def test_kept_set_is_the_max_sum_subset(n, k, rng):
    nh, hd = 1, 64
    c = _cache(rng, nh, hd, n, n - 1)
    qkv = rng.normal(size=(1, 3 * hd)).astype(F16)
    sp = (k - 0.5) / n                          # ceil(sp * n) = k
    assert O.topk_count(sp, n) == k
    out = O.attn_decode(qkv, n - 1, c, sparsity=sp)
    s = _scores(c, qkv[0, :hd], n - 1, 0)
    _, vh = c.read(0, 0, n)
    best = max(itertools.combinations(range(n), k), key=lambda sub: s[list(sub)].sum())
    sub = list(best)
    w = np.exp(s[sub] - s[sub].max())
    ref = (w / w.sum()) @ vh[sub]
    assert np.array_equal(out[0], ref.astype(F16))


def test_equal_scores_keep_the_lower_position(rng):
    nh, hd, S = 1, 64, 6
    c = O.KVCache(1, nh, hd, S + 1)
    k = rng.normal(size=(nh, S, hd)).astype(F16) * F16(0.01)
    big = rng.normal(size=hd).astype(F16)
    for t in (1, 3, 4):
        k[0, t] = big                            # three positions with the same key
    v = rng.normal(size=(nh, S, hd)).astype(F16)
    c.store(0, 0, k, v)
    qkv = np.zeros((1, 3 * hd), F16)
    qkv[0, :hd] = big                            # q . big dominates
    qkv[0, hd:2 * hd] = k[0, 0]                  # the new key: small
    out = O.attn_decode(qkv, S, c, sparsity=1.5 / (S + 1))   # k = 2: positions 1 and 3
    _, vh = c.read(0, 0, S + 1)
    assert np.array_equal(out[0], ((vh[1] + vh[3]) / 2).astype(F16))


def test_dense_limit_and_padding(rng):
    nh, hd, S = 2, 128, 20
    c1 = _cache(rng, nh, hd, S + 1, S)
    c2 = O.KVCache(1, nh, hd, S + 1)
    for a in ("k_codes", "v_codes", "k_params", "v_params"):
        getattr(c2, a)[...] = getattr(c1, a)
    qkv = rng.normal(size=(1, 3 * nh * hd)).astype(F16)
    assert np.array_equal(O.attn_decode(qkv, S, c1), O.attn_decode(qkv, S, c2, sparsity=1.0))
    # with 12 pad positions, 9 real ones compete: sparsity 1/3 keeps 3 of them
    c1.pad[0] = 12
    c3 = O.KVCache(1, nh, hd, S + 1 - 12)
    for a in ("k_codes", "v_codes", "k_params", "v_params"):
        getattr(c3, a)[:, :, :S - 12] = getattr(c2, a)[:, :, 12:S]
    got = O.attn_decode(qkv, S, c1, sparsity=1 / 3)
    ref = O.attn_decode(qkv, S - 12, c3, sparsity=1 / 3)
    assert np.array_equal(got, ref)


def test_generate_with_full_sparsity_is_dense(rng):
    from tests.test_oracle_model import _tiny_model
    m = _tiny_model(rng, L=1, h=128, nh=2, f=256, V=100)
    tok = rng.integers(0, 100, size=(2, 6))
    assert np.array_equal(m.generate(tok, 4, sparsity=1.0), m.generate(tok, 4))
    # one kept position per query: still a valid generation of the right shape
    out = m.generate(tok, 4, sparsity=1e-6)
    assert out.shape == (2, 4) and out.min() >= 0 and out.max() < 100
