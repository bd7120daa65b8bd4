"""Exact rational arithmetic with explicit rounding, for pinning the oracle.

Independent of the oracle's C code: values are Python Fractions and rounding
to a binary format is done here from the format's definition (precision p
including the leading bit, minimum normal exponent emin, maximum exponent emax,
round to nearest with ties to even, gradual underflow, overflow to infinity).
"""
from fractions import Fraction
import math
import struct

import numpy as np

FORMATS = {"f32": (24, -126, 127), "f16": (11, -14, 15), "bf16": (8, -126, 127)}
INF = float("inf")


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_to(x, fmt):
    """Round an exact rational (or +-inf) to format `fmt`; returns Fraction or +-inf."""
    if isinstance(x, float) and math.isinf(x):
        return x
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    p, emin, emax = FORMATS[fmt]
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = max(_floor_log2(a), emin)
    ulp = Fraction(2) ** (e - p + 1)
    q = a / ulp
    n = q.numerator // q.denominator
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    res = n * ulp
    if res >= Fraction(2) ** (emax + 1):
        return sign * INF
    return sign * res


def sqrt_rounded(x, fmt):
    """Correctly rounded square root of a non-negative rational."""
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    s = 64
    while True:
        scaled = x * Fraction(4) ** s
        n = scaled.numerator // scaled.denominator
        r = math.isqrt(n)
        lo = Fraction(r, 2 ** s)
        if r * r == n and scaled.denominator == 1:
            return round_to(lo, fmt)
        hi = Fraction(r + 1, 2 ** s)
        a, b = round_to(lo, fmt), round_to(hi, fmt)
        if a == b:
            return a
        s += 32


def f32(x) -> Fraction:
    """Exact value of a finite fp32 number."""
    return Fraction(float(np.float32(x)))


def to_np32(x) -> np.float32:
    if isinstance(x, float):
        return np.float32(x)
    v = np.float32(float(x))
    assert Fraction(float(v)) == x, "value is not an fp32 number"
    return v


def bits32(x: np.float32) -> int:
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]
