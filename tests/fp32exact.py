"""Exact-arithmetic helpers for the oracle pins (no method arithmetic)."""
from fractions import Fraction
from decimal import Decimal, getcontext

import numpy as np


def round_f32(q: Fraction) -> np.float32:
    """Round an exact rational to binary32, ties to even (normal range only)."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    # q in [2^e, 2^(e+1)); 24-bit significand
    scaled = q / (Fraction(2) ** (e - 23))
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return np.float32(sign * float(Fraction(m) * Fraction(2) ** (e - 23)))


def ln2_fraction(digits=60) -> Fraction:
    getcontext().prec = digits
    return Fraction(Decimal(2).ln())


def gamma(n: int) -> float:
    u = 2.0 ** -24
    return n * u / (1 - n * u)


def r64_bound(L: int) -> float:
    """Relative error factor of the 64-way strided fma reduction: each term
    passes through ceil(L/64) fused multiply-adds and 6 additions."""
    return gamma(-(-L // 64) + 6)
