"""Exact/high-precision references used to pin the oracle (test-only).

Nothing here calls the oracle: values are built from Python's Fraction and
Decimal so that a mistake in the oracle's C arithmetic (a dropped term, a
wrong sign, a wrong rounding rule) shows up as a mismatch.
"""
from __future__ import annotations

import decimal
from fractions import Fraction

import numpy as np

CTX = decimal.Context(prec=60)


def bf16_bits_to_fraction(b: int) -> Fraction:
    f = np.array([int(b) << 16], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(f))


def fraction_to_bf16_bits(x: Fraction) -> int:
    """Round an exact rational to bf16 (8 significant bits), ties to even."""
    if x == 0:
        return 0
    sign = 1 if x < 0 else 0
    a = -x if x < 0 else x
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e - 7, -133)
    scaled = a / (Fraction(2) ** q)
    r = round(scaled)                      # Fraction.__round__: ties to even
    val = Fraction(r) * (Fraction(2) ** q)
    if val >= Fraction(2) ** 128:
        return 0xFF80 if sign else 0x7F80
    f32 = np.array([float(val)], dtype=np.float32)
    assert Fraction(float(f32[0])) == val
    bits = int(f32.view(np.uint32)[0] >> 16)
    return bits | (0x8000 if sign else 0)


def near_bf16_tie(x: Fraction, rel: float = 1e-12) -> bool:
    """True when x lies within rel of a bf16 rounding boundary (midpoint)."""
    if x == 0:
        return False
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e - 7, -133)
    scaled = a / (Fraction(2) ** q)
    frac = scaled - (scaled.numerator // scaled.denominator)
    return abs(frac - Fraction(1, 2)) < Fraction(rel) * scaled


def dec(x) -> decimal.Decimal:
    if isinstance(x, Fraction):
        return CTX.divide(decimal.Decimal(x.numerator), decimal.Decimal(x.denominator))
    return decimal.Decimal(x)


def dec_to_fraction(d: decimal.Decimal) -> Fraction:
    return Fraction(d)
