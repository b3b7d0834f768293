"""Pins for the oracle's 4-bit linear layer and LayerNorm (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import flexq_oracle as O
from tests.oracle_helpers import F16, exact_dot, grid_matrix, nearest_f16


def test_grid_weights_quantize_exactly(rng):
    w16, c, s, off = grid_matrix(rng, 24, 320)
    codes, params = O.quantize(w16)
    assert np.array_equal(O.unpack_nibbles(codes), c)
    assert np.array_equal(params[..., 1].astype(np.float64), s)
    assert np.array_equal(params[..., 0].astype(np.float64), off)
    assert np.array_equal(O.dequantize_weight(codes, params).view(np.uint16), w16.view(np.uint16))


@pytest.mark.parametrize("relu,use_res", [(False, False), (True, False), (False, True), (True, True)])
def test_linear_matches_exact_rational_product(rng, relu, use_res):
    # M, N, K all different so any transposed operand fails
    M, N, K = 3, 5, 192
    w16, *_ = grid_matrix(rng, N, K)
    x = rng.normal(size=(M, K)).astype(F16)
    b = (rng.normal(size=N) * 0.3).astype(F16)
    res = rng.normal(size=(M, N)).astype(F16) if use_res else None
    y = O.linear_w4(x, *O.quantize(w16), bias=b, residual=res, relu=relu)
    assert y.shape == (M, N) and y.dtype == F16
    for m in range(M):
        for n in range(N):
            acc = exact_dot(x[m], w16[n]) + Fraction(float(b[n]))
            if relu and acc < 0:
                acc = Fraction(0)
            if use_res:
                acc += Fraction(float(res[m, n]))
            assert y[m, n].view(np.uint16) == nearest_f16(acc).view(np.uint16), (m, n)


def test_linear_single_code_rows_closed_form(rng):
    # row n holds 15 at column n and 0 elsewhere: step 1, codes exact -> y = 15 x[:, n] + b
    N, K, M = 64, 128, 7
    w16 = np.zeros((N, K), F16)
    w16[np.arange(N), np.arange(N)] = 15
    x = rng.normal(size=(M, K)).astype(F16)
    b = rng.normal(size=N).astype(F16)
    y = O.linear_w4(x, *O.quantize(w16), bias=b)
    want = (15 * x[:, :N].astype(np.float64) + b.astype(np.float64)).astype(F16)
    assert np.array_equal(y.view(np.uint16), want.view(np.uint16))


def test_linear_constant_weight_closed_form(rng):
    # every weight equal to w0: step 0, all codes 0 -> y = w0 * sum_k x + b
    N, K, M = 9, 256, 4
    w0 = F16(0.375)
    codes, params = O.quantize(np.full((N, K), w0, F16))
    assert np.all(codes == 0) and np.all(params[..., 1] == 0)
    x = (rng.integers(-8, 8, size=(M, K)) / 8).astype(F16)    # sums are exact
    y = O.linear_w4(x, codes, params, bias=np.full(N, 1.0, F16))
    want = (x.astype(np.float64).sum(1, keepdims=True) * 0.375 + 1.0) * np.ones((1, N))
    assert np.array_equal(y, want.astype(F16))


def test_logits_output_is_not_rounded(rng):
    w16, *_ = grid_matrix(rng, 6, 128)
    x = rng.normal(size=(2, 128)).astype(F16)
    y = O.linear_w4(x, *O.quantize(w16), out_dtype=np.float64)
    for m in range(2):
        for n in range(6):
            assert abs(Fraction(float(y[m, n])) - exact_dot(x[m], w16[n])) < Fraction(1, 2**40)


def test_sampled_linear_agrees_with_full(rng):
    N, K, M = 40, 256, 6
    w = (rng.normal(size=(N, K)) * 0.02).astype(F16)
    codes, params = O.quantize(w)
    x = rng.normal(size=(M, K)).astype(F16)
    b = rng.normal(size=N).astype(F16)
    r = rng.normal(size=(M, N)).astype(F16)
    full = O.linear_w4(x, codes, params, bias=b, residual=r, relu=True)
    rows = rng.integers(0, M, 30)
    cols = rng.integers(0, N, 30)
    samp = O.linear_w4_sampled(x, codes, params, rows, cols, bias=b, residual=r, relu=True)
    assert np.array_equal(samp.view(np.uint16), full[rows, cols].view(np.uint16))


# ----------------------------------------------------------------- LayerNorm

def test_layernorm_constant_row_gives_beta(rng):
    h = 256
    x = np.full((3, h), 2.75, F16)
    g = rng.normal(size=h).astype(F16)
    b = rng.normal(size=h).astype(F16)
    assert np.array_equal(O.layernorm(x, g, b).view(np.uint16), b[None].repeat(3, 0).view(np.uint16))


def test_layernorm_two_level_row_closed_form(rng):
    # mean 0, biased variance a^2 -> +-a / sqrt(a^2 + 1e-5) * g + beta
    h = 128
    for a in (0.001, 0.5, 3.0, 100.0):
        x = np.where(np.arange(h) % 2 == 0, a, -a).astype(F16)[None]
        g = rng.normal(size=h).astype(F16)
        be = rng.normal(size=h).astype(F16)
        a16 = float(F16(a))
        z = np.where(np.arange(h) % 2 == 0, 1.0, -1.0) * a16 / np.sqrt(a16 * a16 + 1e-5)
        want = (z * g.astype(np.float64) + be.astype(np.float64)).astype(F16)
        got = O.layernorm(x, g, be)[0]
        ulp = np.abs(np.spacing(want.astype(np.float32)))
        assert np.all(np.abs(got.astype(np.float64) - want.astype(np.float64)) <= ulp)


def test_layernorm_normalises_moments(rng):
    h = 2048
    x = (rng.normal(size=(8, h)) * 7 + 3).astype(F16)
    y = O.layernorm(x, np.ones(h, F16), np.zeros(h, F16)).astype(np.float64)
    assert np.all(np.abs(y.mean(1)) < 2e-3)
    assert np.all(np.abs(y.std(1) - 1) < 2e-3)
    # shift invariance on rows where the shift is exact in fp16
    xi = (rng.integers(-64, 64, size=(4, h)) / 8).astype(F16)
    ya = O.layernorm(xi, np.ones(h, F16), np.zeros(h, F16)).astype(np.float64)
    yb = O.layernorm((xi.astype(np.float64) + 16).astype(F16), np.ones(h, F16),
                     np.zeros(h, F16)).astype(np.float64)
    assert np.all(np.abs(ya - yb) <= np.abs(np.spacing(ya.astype(np.float16))).astype(np.float64))
