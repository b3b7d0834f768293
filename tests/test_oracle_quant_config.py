"""Pins of the oracle's general-config quantizer (`quantize_config`): bit packing by
closed form, exact ramps, brute-force nearest codes, the round-to-nearest error bound,
padded tails, the grouped axis, and the 4-bit default against the pages' packed
shape and the 4-bit quantizer."""
import numpy as np
import pytest

from oracle import flexq_oracle as O

F16 = np.float16
BITS = range(2, 9)


@pytest.mark.parametrize("b", BITS)
def test_pack_bits_single_code_sets_exactly_its_bits(b):
    n = 8 * 3          # n * b is a multiple of 8 for every b
    for i in range(n):
        c = np.zeros(n, np.uint16)
        c[i] = (1 << b) - 1
        stream = O.pack_bits(c, b)
        bits = np.unpackbits(stream, bitorder="little")
        want = np.zeros(n * b, np.uint8)
        want[b * i:b * i + b] = 1
        assert np.array_equal(bits, want), (b, i)


@pytest.mark.parametrize("b", BITS)
def test_pack_unpack_round_trip(b, rng):
    c = rng.integers(0, 1 << b, size=(5, 64)).astype(np.uint16)
    assert np.array_equal(O.unpack_bits(O.pack_bits(c, b), b), c)


def test_pack_bits_4_is_the_nibble_order():
    c = np.arange(64, dtype=np.uint16) % 16
    assert np.array_equal(O.pack_bits(c, 4), O.pack_nibbles(c.astype(np.uint8)))
    assert np.array_equal(O.pack_bits(np.arange(16, dtype=np.uint16) * 16 % 256, 8),
                          (np.arange(16) * 16 % 256).astype(np.uint8))


@pytest.mark.parametrize("b", BITS)
def test_asymmetric_ramp_is_exact(b):
    # values m + k d with integers k from 0 to 2^b - 1 (both ends present): step d,
    # offset m, codes k
    q = (1 << b) - 1
    m, d = -3.0, 0.25
    k = (np.arange(64) * q) // 63
    x = (m + k * d).astype(F16)[None, :]
    assert np.all(x.astype(np.float64) == m + k * d)
    codes, params = O.quantize_config(x, b, 64)
    assert params[0, 0, 0] == F16(m) and params[0, 0, 1] == F16(d)
    assert np.array_equal(O.unpack_bits(codes, b)[0], k)


@pytest.mark.parametrize("b", BITS)
def test_symmetric_ramp_is_exact(b):
    B = (1 << (b - 1)) - 1
    d = 0.5
    k = (np.arange(64) * 2 * B) // 63 - B          # integers from -B to B, both ends present
    x = (k * d).astype(F16)[None, :]
    codes, params = O.quantize_config(x, b, 64, symmetric=True)
    assert params[0, 0, 1] == F16(d) and params[0, 0, 0] == F16(0)
    assert np.array_equal(O.unpack_bits(codes, b)[0].astype(np.int64), k + (1 << (b - 1)))


@pytest.mark.parametrize("b", BITS)
@pytest.mark.parametrize("sym", [False, True])
def test_codes_are_nearest_within_step_half(b, sym, rng):
    x = (rng.normal(size=(40, 64)) * 2.0 ** rng.integers(-6, 6, size=(40, 1))).astype(F16)
    codes, params = O.quantize_config(x, b, 64, symmetric=sym)
    c = O.unpack_bits(codes, b).astype(np.int64)
    s = params[:, 0, 1].astype(np.float64)[:, None]
    off = params[:, 0, 0].astype(np.float64)[:, None]
    if sym:
        levels = np.arange(1, 1 << b) - (1 << (b - 1))            # -B .. B
        val = (c - (1 << (b - 1))) * s
    else:
        levels = np.arange(1 << b)
        val = c * s + off
    cand = levels[None, None, :] * s[:, :, None] + (0 if sym else off[:, :, None])
    dist = np.abs(x.astype(np.float64)[:, :, None] - cand)
    chosen = np.abs(x.astype(np.float64) - val)
    # brute force over every representable level; fp32 decisions may pick a neighbour
    # only at a near tie (a few fp32 ulps of the scaled value)
    assert np.all(chosen <= dist.min(axis=2) + s * 2.0**-15)
    # and the error is within half a step (plus the fp16 rounding of the step itself)
    assert np.all(chosen <= s / 2 * (1 + 2.0**-9) + 1e-30)
    v = O.dequantize_config(codes, params, 64, b, 64, symmetric=sym)
    assert np.array_equal(v, val)


@pytest.mark.parametrize("sym", [False, True])
def test_constant_group(sym):
    x = np.full((1, 64), 0.0 if sym else 1.5, F16)
    codes, params = O.quantize_config(x, 3, 64, symmetric=sym)
    assert params[0, 0, 1] == 0
    c = O.unpack_bits(codes, 3)[0]
    assert np.all(c == (4 if sym else 0))
    assert np.array_equal(O.dequantize_config(codes, params, 64, 3, 64, symmetric=sym)[0],
                          x[0].astype(np.float64))


def test_padded_tail_takes_part_as_zeros():
    # 100 values in [1, 2]: the second group has 36 of them and 28 zeros of padding,
    # so its minimum (the offset) is 0; the first group's is its own minimum
    x = np.linspace(1.0, 2.0, 100).astype(F16)[None, :]
    codes, params = O.quantize_config(x, 4, 64)
    assert codes.shape == (1, 2 * 32) and params.shape == (1, 2, 2)
    assert params[0, 1, 0] == 0 and params[0, 0, 0] == x[0, 0]
    assert params[0, 1, 1] == F16(np.float32(x[0, 99]) / np.float32(15))
    c = O.unpack_bits(codes, 4)[0]
    assert np.all(c[100:] == 0)
    v = O.dequantize_config(codes, params, 100, 4, 64)
    assert v.shape == (1, 100)


@pytest.mark.parametrize("b,g,sym", [(3, 64, False), (5, 32, True), (8, 16, False), (2, 128, True)])
def test_group_dim_is_the_same_as_quantizing_each_slice(b, g, sym, rng):
    x = rng.normal(size=(3, 130, 5)).astype(F16)
    codes, params = O.quantize_config(x, b, g, group_dim=1, symmetric=sym)
    ng = -(-130 // g)
    assert codes.shape == (3, ng * g * b // 8, 5) and params.shape == (3, ng, 5, 2)
    for o in range(3):
        for i in range(5):
            c1, p1 = O.quantize_config(x[o, :, i][None, :], b, g, symmetric=sym)
            assert np.array_equal(codes[o, :, i], c1[0])
            assert np.array_equal(params[o, :, i].view(np.uint16), p1[0].view(np.uint16))


def test_default_config_is_the_4bit_path(rng):
    x = rng.normal(size=(6, 256)).astype(F16)
    c1, p1 = O.quantize(x)
    c2, p2 = O.quantize_config(x)
    assert np.array_equal(c1, c2) and np.array_equal(p1.view(np.uint16), p2.view(np.uint16))


@pytest.mark.parametrize("b,g", [(1, 64), (9, 64), (3, 4), (5, 12)])
def test_rejects_unsupported_configs(b, g):
    with pytest.raises(ValueError):
        O.quantize_config(np.zeros((2, 64), F16), b, g)
