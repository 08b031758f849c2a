"""Exact-arithmetic helpers for pinning the oracle (no part of the oracle).

Everything here is done in Python integers / fractions, so it is independent of
the C oracle's floating-point evaluation order.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def exact_abs_sum(W: np.ndarray) -> Fraction:
    """Exact sum of |W| for a float32 array, as a Fraction."""
    a = np.abs(np.asarray(W, dtype=np.float32)).ravel().astype(np.float64)
    a = a[a != 0.0]
    if a.size == 0:
        return Fraction(0)
    m, e = np.frexp(a)  # a = m * 2**e, 0.5 <= m < 1, exact for float32 values
    mi = (m * (1 << 24)).astype(np.int64)  # 24-bit integer significand
    assert np.all(mi.astype(np.float64) == m * (1 << 24))
    # each value is mi * 2**(ex - 24); shift every term by 2**SHIFT so that
    # all exponents become non-negative integers (float32 needs ex - 24 >= -173)
    SHIFT = 200
    total = 0
    for ex in np.unique(e):
        s = int(mi[e == ex].sum())
        total += s << int(ex - 24 + SHIFT)
    return Fraction(total, 1 << SHIFT)


def round_to_f32(q: Fraction) -> np.float32:
    """Round a non-negative rational to the nearest float32, ties to even."""
    if q == 0:
        return np.float32(0.0)
    assert q > 0
    # exponent e with 2**e <= q < 2**(e+1)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    assert Fraction(2) ** e <= q < Fraction(2) ** (e + 1)
    assert e >= -126, "subnormal results are not needed here"
    scaled = q * Fraction(2) ** (23 - e)  # in [2**23, 2**24)
    mant = scaled.numerator // scaled.denominator
    rem = scaled - mant
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and (mant & 1)):
        mant += 1
    return np.float32(float(Fraction(mant) * Fraction(2) ** (e - 23)))


def f32_ulp(x: np.float32) -> float:
    x = np.float32(x)
    return float(np.nextafter(x, np.float32(np.inf)) - x)
