"""Test-side input builders for the oracle pins (no method arithmetic).

`grid_matrix` builds fp16 matrices whose every 64-group is exactly representable by
the 4-bit code: step a power of two, offset a multiple of it, codes 0 and 15 both
present.  Quantizing such a matrix must give back exactly those steps, offsets and
codes, so tests can compare against library routines on the original fp16 values.
"""
from fractions import Fraction

import numpy as np

F16 = np.float16


def grid_matrix(rng, rows, cols, emin=-9, emax=-4):
    g = cols // 64
    e = rng.integers(emin, emax + 1, size=(rows, g, 1))
    s = np.ldexp(1.0, e)
    k = rng.integers(-40, 25, size=(rows, g, 1))
    c = rng.integers(0, 16, size=(rows, g, 64))
    c[..., 0] = 0
    c[..., 1] = 15
    c = rng.permuted(c, axis=2)
    w = ((k + c) * s).reshape(rows, cols)
    w16 = w.astype(F16)
    assert np.array_equal(w16.astype(np.float64), w)
    return w16, c.reshape(rows, cols).astype(np.uint8), s.reshape(rows, g), (k * s).reshape(rows, g)


def nearest_f16(q: Fraction):
    return np.float64(float(q)).astype(F16)


def exact_dot(a, b):
    return sum((Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a, b)), Fraction(0))
