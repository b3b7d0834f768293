"""Closed-form pins for three oracle steps that the random-input pins leave open (CPU only).

* the quantizer's tie rule: scaled values that land exactly halfway between two
  codes (reading of the walkthrough's section 6.3, which fixes 4-bit min/max groups
  but no rounding rule: round half to even);
* the attention half of a pre-LN layer (source notes "Flex Opt": embedding, N
  transformer layers, output head): at one prompt token the attention returns v
  itself, so the half is x + Wo (Wv LN1(x) + bv) + bo in exact arithmetic, with
  LN1's parameters and not LN2's;
* the position each generated token is embedded at (walkthrough section 4.1,
  `generate`): a model whose layers are all zero passes the embedding straight to
  the output head, so a positional table that points at one token per row makes
  every generated token name the position it was embedded at.
"""
from fractions import Fraction

import numpy as np

from oracle import flexq_oracle as O
from tests.oracle_helpers import F16, exact_dot, grid_matrix, nearest_f16


# ----------------------------------------------------------------- ties round half to even

def _step_one_group(lo, values):
    """A 64-group with minimum lo and maximum lo + 15 (step exactly 1) holding `values`."""
    g = np.full(64, lo + 7.0)
    g[0], g[1] = lo, lo + 15.0
    g[2:2 + len(values)] = values
    return g.astype(F16)


def test_quantizer_ties_go_to_the_even_code():
    # (x - min) * (1 / step) = k + 1/2 exactly: the even neighbour wins
    halves = np.array([0.5, 1.5, 2.5, 3.5, 6.5, 7.5, 13.5, 14.5])
    even = np.array([0, 2, 2, 4, 6, 8, 14, 14])
    for lo in (0.0, -8.0, 32.0, -1024.0):
        g = _step_one_group(lo, lo + halves)
        assert np.array_equal(g[2:2 + halves.size].astype(np.float64), lo + halves)
        codes, params = O.quantize(g[None, :])
        assert float(params[0, 0, 1]) == 1.0 and float(params[0, 0, 0]) == lo
        c = O.unpack_nibbles(codes)[0]
        assert np.array_equal(c[2:2 + halves.size], even), lo
        assert c[0] == 0 and c[1] == 15


def test_quantizer_near_ties_go_to_the_nearer_code():
    # one fp16 ulp either side of the tie decides by distance, not by parity
    lo = 0.0
    vals = np.array([2.5 - 2**-8, 2.5 + 2**-8, 13.5 - 2**-7, 13.5 + 2**-7])
    g = _step_one_group(lo, vals)
    c = O.unpack_nibbles(O.quantize(g[None, :])[0])[0]
    assert list(c[2:6]) == [2, 3, 13, 14]


# ----------------------------------------------------------------- attention half uses LN1

def _attention_half_layer(rng, h, f):
    w = dict(ln1_g=(2.0 + rng.normal(size=h) * 0.25).astype(F16),
             ln1_b=(0.5 + rng.normal(size=h) * 0.25).astype(F16),
             ln2_g=(0.5 + rng.normal(size=h) * 0.1).astype(F16),
             ln2_b=(-1.0 + rng.normal(size=h) * 0.1).astype(F16),
             wqkv=grid_matrix(rng, 3 * h, h, emin=-7, emax=-5)[0],
             bqkv=(rng.normal(size=3 * h) * 0.1).astype(F16),
             wo=grid_matrix(rng, h, h, emin=-7, emax=-5)[0],
             bo=(rng.normal(size=h) * 0.1).astype(F16),
             # the feed-forward half is zero: x2 = x1 + fp16(0) exactly
             w1=np.zeros((f, h), F16), b1=np.zeros(f, F16),
             w2=np.zeros((h, f), F16), b2=np.zeros(h, F16))
    return w


def _attention_half_exact(w, x, h):
    """x1 = fp16(x + Wo v + bo), v = fp16(Wv a + bv), a = LN1(x): exact sums, one rounding each."""
    a = O.layernorm(x[None, :], w["ln1_g"], w["ln1_b"])[0]
    v = [nearest_f16(exact_dot(a, w["wqkv"][2 * h + n]) + Fraction(float(w["bqkv"][2 * h + n])))
         for n in range(h)]
    return np.array([nearest_f16(exact_dot(v, w["wo"][n]) + Fraction(float(w["bo"][n]))
                                 + Fraction(float(x[n]))) for n in range(h)], F16)


def test_attention_half_is_x_plus_out_of_v_of_ln1(rng):
    h, f, nh = 128, 256, 2
    w = _attention_half_layer(rng, h, f)
    L = O.QLayer(w, nh)
    x = (rng.normal(size=(2, h)) * 2).astype(F16)
    # prefill of one-token prompts: each query sees only its own key, p = 1, out = v
    y = L.prefill(x, 2, 1, O.KVCache(2, nh, h // nh, 2))
    for b in range(2):
        want = _attention_half_exact(w, x[b], h)
        assert np.array_equal(y[b].view(np.uint16), want.view(np.uint16)), b
    # the same structure with LN2's parameters in the attention half would differ
    w_swapped = dict(w, ln1_g=w["ln2_g"], ln1_b=w["ln2_b"])
    assert not np.array_equal(_attention_half_exact(w_swapped, x[0], h), y[0])


def test_decode_attention_half_over_one_cached_token(rng):
    # decode at position 0 of an empty cache: the token attends only to itself, read
    # back from the 4-bit cache; with v a grid of one step per 64-group the dequantized
    # v equals the fp16 v, so the closed form above holds at decode too
    h, f, nh = 128, 256, 2
    w = _attention_half_layer(rng, h, f)
    # V rows of wqkv zero, V bias on a grid: v = bv for any input, and bv quantizes exactly
    w["wqkv"][2 * h:] = 0
    bv = grid_matrix(rng, 1, h, emin=-6, emax=-6)[0][0]
    w["bqkv"][2 * h:] = bv
    L = O.QLayer(w, nh)
    x = (rng.normal(size=(1, h)) * 2).astype(F16)
    y = L.decode(x, 0, O.KVCache(1, nh, h // nh, 1))
    assert np.array_equal(y[0].view(np.uint16), _attention_half_exact(w, x[0], h).view(np.uint16))


# ----------------------------------------------------------------- decode positions

V_POS, H_POS, AMP_E, AMP_P = 64, 64, 0.9375, 8.0


def _pointer_token(row):
    """The token that positional row `row` points at."""
    return (5 * row + 3) % V_POS


def _pointer_model(layers=2, nh=1):
    h, f = H_POS, 128
    zero = dict(ln1_g=np.ones(h, F16), ln1_b=np.zeros(h, F16), ln2_g=np.ones(h, F16),
                ln2_b=np.zeros(h, F16), wqkv=np.zeros((3 * h, h), F16),
                bqkv=np.zeros(3 * h, F16), wo=np.zeros((h, h), F16), bo=np.zeros(h, F16),
                w1=np.zeros((f, h), F16), b1=np.zeros(f, F16), w2=np.zeros((h, f), F16),
                b2=np.zeros(h, F16))
    # token t: AMP_E at column t (one group of 64: min 0, max 15/16, step 1/16 exactly)
    emb = (np.eye(V_POS, h) * AMP_E).astype(F16)
    # positional row r: AMP_P at column _pointer_token(r)
    pos = np.zeros((2050, h), F16)
    pos[np.arange(2050), _pointer_token(np.arange(2050))] = AMP_P
    return O.QModel([O.QLayer(zero, nh) for _ in range(layers)], emb, pos, np.ones(h, F16),
                    np.zeros(h, F16), nh), emb, pos


def test_zero_layers_pass_the_embedding_to_the_head():
    model, emb, pos = _pointer_model()
    codes, params = O.quantize(emb)
    assert np.array_equal(O.dequantize_weight(codes, params), emb)
    caches = model.new_caches(1, 8)
    tok, p = 17, 5
    logits, nxt = model.decode_step(np.array([tok]), p, caches)
    x = (emb[tok].astype(np.float64) + pos[p + 2].astype(np.float64)).astype(F16)
    want = O.layernorm(x[None, :], np.ones(H_POS, F16), np.zeros(H_POS, F16)).astype(np.float64)
    assert np.allclose(logits, AMP_E * want, rtol=0, atol=1e-12)
    assert nxt[0] == _pointer_token(p + 2)


def test_generated_tokens_follow_prompt_length_and_padding(rng):
    # prompt length S; the prefill's token follows position S - 1 - pad, decode step i
    # embeds its input at position S + i - pad
    model, _, _ = _pointer_model()
    S, G = 7, 5
    toks = rng.integers(0, V_POS, size=(3, S))
    pad = np.array([0, 2, 6])
    out = model.generate(toks, G, pad=pad)
    for b in range(3):
        want = [_pointer_token(S - 1 - pad[b] + 2)] + \
               [_pointer_token(S + i - pad[b] + 2) for i in range(G - 1)]
        assert list(out[b]) == want, (b, list(out[b]), want)
