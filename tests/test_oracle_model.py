"""Pins for the oracle's OPT layer, embedding, output head and greedy loop (CPU only)."""
from fractions import Fraction

import numpy as np

from oracle import flexq_oracle as O
from tests.oracle_helpers import F16, exact_dot, grid_matrix, nearest_f16


def _layer_w16(rng, h, f, zero_mats=False, scale=0.05):
    def mat(n, k):
        return np.zeros((n, k), F16) if zero_mats else (rng.normal(size=(n, k)) * scale).astype(F16)

    def vec(n, mean=0.0):
        return (mean + rng.normal(size=n) * 0.1).astype(F16)

    return dict(ln1_g=vec(h, 1), ln1_b=vec(h), wqkv=mat(3 * h, h), bqkv=vec(3 * h),
                wo=mat(h, h), bo=vec(h), ln2_g=vec(h, 1), ln2_b=vec(h),
                w1=mat(f, h), b1=vec(f), w2=mat(h, f), b2=vec(h))


def test_zero_weight_layer_is_residual_plus_biases(rng):
    # all matrices 0: attention/FFN contribute only their output biases
    # x1 = fp16(x + bo), x2 = fp16(x1 + b2)   (W2 relu(b1) = 0)
    h, f, nh, B, S = 128, 512, 2, 2, 5
    w = _layer_w16(rng, h, f, zero_mats=True)
    L = O.QLayer(w, nh)
    x = rng.normal(size=(B * S, h)).astype(F16)
    cache = O.KVCache(B, nh, h // nh, S + 1)
    y = L.prefill(x, B, S, cache)
    x1 = (x.astype(np.float64) + w["bo"].astype(np.float64)).astype(F16)
    want = (x1.astype(np.float64) + w["b2"].astype(np.float64)).astype(F16)
    assert np.array_equal(y.view(np.uint16), want.view(np.uint16))
    yd = L.decode(x[:B], S, cache)
    x1d = (x[:B].astype(np.float64) + w["bo"].astype(np.float64)).astype(F16)
    assert np.array_equal(yd, (x1d.astype(np.float64) + w["b2"].astype(np.float64)).astype(F16))


def test_layer_is_pre_ln_with_relu_ffn(rng):
    # attention half zeroed (wqkv = wo = 0); FFN half exact grid weights:
    # y = x1 + W2 relu(W1 LN2(x1) + b1) + b2 checked element-wise in exact arithmetic
    h, f, nh, B, S = 64, 128, 1, 1, 3
    w = _layer_w16(rng, h, f, zero_mats=True)
    w["w1"] = grid_matrix(rng, f, h, emin=-6, emax=-5)[0]
    w["w2"] = grid_matrix(rng, h, f, emin=-7, emax=-6)[0]
    L = O.QLayer(w, nh)
    x = rng.normal(size=(B * S, h)).astype(F16)
    y = L.prefill(x, B, S, O.KVCache(B, nh, h, S))
    x1 = (x.astype(np.float64) + w["bo"].astype(np.float64)).astype(F16)
    a = O.layernorm(x1, w["ln2_g"], w["ln2_b"])
    for m in range(B * S):
        u = []
        for n in range(f):
            acc = exact_dot(a[m], w["w1"][n]) + Fraction(float(w["b1"][n]))
            u.append(nearest_f16(max(acc, Fraction(0))))
        for n in range(h):
            acc = exact_dot(u, w["w2"][n]) + Fraction(float(w["b2"][n])) + Fraction(float(x1[m, n]))
            assert y[m, n].view(np.uint16) == nearest_f16(acc).view(np.uint16), (m, n)


def test_embedding_adds_position_row_with_offset_two(rng):
    V, h = 40, 128
    e16 = grid_matrix(rng, V, h)[0]
    codes, params = O.quantize(e16)
    pos = (np.arange(20)[:, None] * np.ones((1, h)) / 4).astype(F16)     # row j = j/4
    toks = np.array([3, 39, 0])
    positions = np.array([0, 5, 17])
    x = O.embed(toks, positions, codes, params, pos)
    want = (e16[toks].astype(np.float64) + ((positions + 2) / 4)[:, None]).astype(F16)
    assert np.array_equal(x, want)


def test_lm_head_logits_and_lowest_index_ties(rng):
    V, h = 96, 128
    e16 = grid_matrix(rng, V, h)[0]
    e16[70] = e16[11]                      # duplicate rows give tied logits
    codes, params = O.quantize(e16)
    x = rng.normal(size=(4, h)).astype(F16)
    g = np.ones(h, F16)
    b = np.zeros(h, F16)
    logits, nxt = O.lm_head(x, g, b, codes, params)
    a = O.layernorm(x, g, b)
    for m in range(4):
        for n in range(V):
            assert abs(Fraction(float(logits[m, n])) - exact_dot(a[m], e16[n])) < Fraction(1, 2**36)
    assert np.array_equal(nxt, logits.argmax(1))
    # force the duplicated row to win: put a on the direction of row 11
    x2 = e16[11][None].astype(F16) * F16(8)
    _, n2 = O.lm_head(x2, g, b, codes, params)
    lg2, _ = O.lm_head(x2, g, b, codes, params)
    if lg2[0, 11] == lg2[0].max():
        assert n2[0] == 11


def _tiny_model(rng, L=2, h=128, nh=2, f=256, V=512):
    layers = [O.QLayer(_layer_w16(rng, h, f), nh) for _ in range(L)]
    emb = (rng.normal(size=(V, h)) * 0.5).astype(F16)
    pos = (rng.normal(size=(2050, h)) * 0.1).astype(F16)
    return O.QModel(layers, emb, pos, np.ones(h, F16), np.zeros(h, F16), nh)


def test_generate_matches_manual_loop_and_is_per_sequence(rng):
    model = _tiny_model(rng)
    B, S, G = 3, 6, 4
    toks = rng.integers(0, 512, size=(B, S))
    out = model.generate(toks, G)
    assert out.shape == (B, G)
    caches = model.new_caches(B, S + G - 1)
    _, nxt = model.prefill(toks, caches)
    manual = [nxt]
    for i in range(G - 1):
        _, nxt = model.decode_step(nxt, S + i, caches)
        manual.append(nxt)
    assert np.array_equal(out, np.stack(manual, 1))
    solo = model.generate(toks[1:2], G)
    assert np.array_equal(solo, out[1:2])
