"""Pins for the oracle's quantizer, packing and dequantizer (CPU only).

Each test checks the oracle against something other than itself: closed forms,
exhaustive enumeration, brute-force nearest-code search, exact rational arithmetic
or the figures the pages print (tests/golden/compression_config.txt).
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import flexq_oracle as O

F16 = np.float16
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "compression_config.txt")


def _golden():
    out = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split("=")
            out[k] = v
    return out


# ----------------------------------------------------------------- fp16 rounding primitive

def test_fp16_rounding_is_single_and_to_even():
    # direct double -> half rounding (no detour through float32)
    assert float(np.float64(1 + 2**-11 + 2**-40).astype(F16)) == 1 + 2**-10
    # exact midpoints go to the even neighbour
    assert float(np.float64(1 + 2**-11).astype(F16)) == 1.0
    assert float(np.float64(1 + 3 * 2**-11).astype(F16)) == 1 + 2**-9
    # subnormals: 2^-25 is the midpoint of 0 and 2^-24 -> 0; 3*2^-26 -> 2^-24
    assert float(np.float64(2**-25).astype(F16)) == 0.0
    assert float(np.float64(3 * 2**-26).astype(F16)) == 2**-24
    assert float(np.float64(65519.99).astype(F16)) == 65504.0


def test_fp16_roundtrip_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    h = bits.view(F16)
    fin = np.isfinite(h)
    back = h[fin].astype(np.float64).astype(F16).view(np.uint16)
    assert np.array_equal(back, bits[fin])


# ----------------------------------------------------------------- nibble packing

def test_pack_unpack_exhaustive():
    b = np.arange(256, dtype=np.uint8)
    c = O.unpack_nibbles(b[None, :])[0]
    assert np.array_equal(c[0::2], b & 15)
    assert np.array_equal(c[1::2], b >> 4)
    assert np.array_equal(O.pack_nibbles(c[None, :])[0], b)


def test_nibble_order():
    # element 2j in the low nibble, element 2j+1 in the high nibble
    assert O.pack_nibbles(np.array([[1, 2, 15, 0]], np.uint8)).tolist() == [[0x21, 0x0F]]


# ----------------------------------------------------------------- quantizer closed forms

def _q1(group):
    codes, params = O.quantize(np.asarray(group, dtype=F16)[None, :])
    return O.unpack_nibbles(codes)[0], params[0, 0]


def test_constant_group():
    c, (off, s) = _q1(np.full(64, 3.5))
    assert np.all(c == 0) and float(s) == 0.0 and float(off) == 3.5
    xh = O.dequantize_exact(O.pack_nibbles(c[None]), np.array([[[off, s]]], F16))
    assert np.all(xh == 3.5)


def test_zero_offset_is_positive_zero():
    g = np.zeros(64, F16)
    g[::2] = F16(-0.0)
    _, (off, s) = _q1(g)
    assert off.view(np.uint16) == 0 and float(s) == 0.0
    g2 = np.linspace(0, 1, 64).astype(F16)
    g2[0] = F16(-0.0)
    _, (off2, _) = _q1(g2)
    assert off2.view(np.uint16) == 0


@pytest.mark.parametrize("a,d", [(-1.5, 0.125), (0.0, 2**-10 * 3), (100.0, 0.5), (-0.0625, 2**-14)])
def test_ramp_group_pins_step_and_order(a, d):
    # x_i = a + (i mod 16) d with every value fp16-exact: step must be d, codes i mod 16
    x = np.array([a + (i % 16) * d for i in range(64)])
    assert np.all(x.astype(F16).astype(np.float64) == x)
    c, (off, s) = _q1(x)
    assert float(s) == d and float(off) == a
    assert np.array_equal(c, np.arange(64) % 16)
    codes, _ = O.quantize(x.astype(F16)[None])
    # bytes j = (2j mod 16) | ((2j+1) mod 16) << 4
    assert codes[0].tolist() == [((2 * j) % 16) | (((2 * j + 1) % 16) << 4) for j in range(32)]


def test_two_valued_group(rng):
    for _ in range(200):
        lo, hi = np.sort(rng.normal(size=2) * 10)
        g = np.where(rng.random(64) < 0.5, lo, hi).astype(F16)
        g[0], g[1] = F16(lo), F16(hi)
        if g[0] == g[1]:
            continue
        c, _ = _q1(g)
        assert set(np.unique(c)) <= {0, 15}
        assert np.all(c[g == g.min()] == 0) and np.all(c[g == g.max()] == 15)


def test_tiny_range_gets_smallest_subnormal_step():
    g = np.zeros(64)
    g[5] = 2**-24
    c, (off, s) = _q1(g)
    assert float(s) == 2**-24 and float(off) == 0.0
    assert c[5] == 1 and np.sum(c) == 1


def _random_groups(rng, n):
    x = rng.normal(size=(n, 64))
    x[: n // 4] *= 8.0 ** rng.integers(-6, 4, size=(n // 4, 1))      # assorted ranges
    x[n // 4: n // 2] += rng.normal(size=(n // 4, 1)) * 100          # far from zero
    m = rng.random(x.shape) < 0.01
    x[m] *= 8                                                         # outliers
    x = x.astype(F16)
    assert np.all(np.isfinite(x))
    return x


def test_error_bound_and_endpoints(rng):
    x = _random_groups(rng, 4000)
    codes, params = O.quantize(x)
    xh = O.dequantize_exact(codes, params)
    c = O.unpack_nibbles(codes)
    s = params[:, 0, 1].astype(np.float64)
    off = params[:, 0, 0].astype(np.float64)
    err = np.abs(x.astype(np.float64) - xh)
    # (x - min)/step within 0.5 of its code, up to three fp32 roundings of a ratio <= 15.01
    assert np.all(err <= s[:, None] * (0.5 + 2.0**-17))
    # the group minimum is reconstructed exactly
    mn = x.min(axis=1).astype(np.float64)
    assert np.array_equal(off, mn)
    assert np.all(c[x.astype(np.float64) == mn[:, None]] == 0)
    # the maximum takes code 15, off by at most 15 x the fp16 rounding error of the step
    # (half an ulp: s * 2^-11 for normal steps, 2^-25 for subnormal ones)
    mx = x.max(axis=1).astype(np.float64)
    cmx = c[np.arange(len(x)), x.argmax(axis=1)]
    assert np.all(cmx == 15)
    half_ulp = np.maximum(s * 2.0**-11, 2.0**-25)
    assert np.all(np.abs(mx - (15 * s + off)) <= 15 * half_ulp + (mx - mn) * 2.0**-22)


def test_codes_are_nearest_brute_force(rng):
    x = _random_groups(rng, 500)
    codes, params = O.quantize(x)
    c = O.unpack_nibbles(codes).astype(np.int64)
    s = params[:, 0, 1].astype(np.float64)[:, None, None]
    off = params[:, 0, 0].astype(np.float64)[:, None, None]
    cand = np.arange(16)[None, None, :] * s + off                       # [n][1][16]
    dist = np.abs(x.astype(np.float64)[:, :, None] - cand)             # [n][64][16]
    chosen = np.take_along_axis(dist, c[:, :, None], axis=2)[:, :, 0]
    assert np.all(chosen <= dist.min(axis=2) + s[:, :, 0] * 2.0**-17)


def test_multi_dim_layout_groups_innermost(rng):
    x = rng.normal(size=(3, 5, 256)).astype(F16)
    codes, params = O.quantize(x)
    assert codes.shape == (3, 5, 128) and params.shape == (3, 5, 4, 2)
    c2, p2 = O.quantize(x.reshape(-1, 64))
    assert np.array_equal(codes.reshape(-1, 32), c2)
    assert np.array_equal(params.reshape(-1, 2), p2.reshape(-1, 2))


def test_rejects_ungrouped_dim():
    with pytest.raises(ValueError):
        O.quantize(np.zeros((2, 96), F16))


# ----------------------------------------------------------------- pages' figures

def test_config_and_packed_shape_match_pages():
    g = _golden()
    assert int(g["weight.num_bits"]) == O.BITS and int(g["weight.group_size"]) == O.GROUP
    assert int(g["cache.num_bits"]) == O.BITS and int(g["cache.group_size"]) == O.GROUP
    assert g["weight.symmetric"] == "False" and g["cache.symmetric"] == "False"
    x = np.zeros((7, 640), F16)
    codes, params = O.quantize(x)
    num_groups = 640 // int(g["weight.group_size"])
    # data_shape = shape[:group_dim] + (num_groups * (group_size // 2),) + ...
    assert codes.shape == (7, num_groups * (int(g["weight.group_size"]) // 2))
    assert codes.dtype == np.uint8


def test_memory_saving_matches_pages():
    g = _golden()
    x = np.zeros((128, 4096), F16)
    codes, params = O.quantize(x)
    per_elem = (codes.nbytes + params.nbytes) / x.size
    assert per_elem == 0.5625
    saving = 1 - per_elem / 2
    assert abs(saving - float(g["weight_memory_saving_approx"])) < 0.03     # 71.9 % ~ 70 %
    assert int(g["opt30b.gpu_batch_size"]) * int(g["opt30b.num_gpu_batches"]) == \
        int(g["opt30b.effective_batch"])


# ----------------------------------------------------------------- dequantization

def test_weight_dequant_is_one_rounding_of_exact_value(rng):
    # exact rational c*s + m, then the nearest fp16 found by neighbour search
    for _ in range(300):
        s = F16(abs(rng.normal()) * 2.0 ** rng.integers(-20, 8))
        m = F16(rng.normal() * 2.0 ** rng.integers(-10, 10))
        for c in range(16):
            codes = O.pack_nibbles(np.full((1, 64), c, np.uint8))
            params = np.array([[[m, s]]], F16)
            got = O.dequantize_weight(codes, params)[0, 0]
            exact = Fraction(c) * Fraction(float(s)) + Fraction(float(m))
            cand = [got, np.nextafter(got, F16(np.inf)), np.nextafter(got, F16(-np.inf))]
            d = [abs(Fraction(float(v)) - exact) for v in cand]
            assert d[0] <= min(d[1:])
            if d[0] == min(d[1:]) and (d[1] == d[0] or d[2] == d[0]):
                assert got.view(np.uint16) % 2 == 0      # tie -> even mantissa
            kv = O.dequantize_kv(codes, params)[0, 0]
            assert Fraction(kv) == exact
