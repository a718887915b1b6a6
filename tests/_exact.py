"""Exact-arithmetic helpers for pinning the oracle (Python ``fractions``).

These are deliberately different methods from the oracle's: rounding to fp32 by
exact rational comparison, and E4M3 encoding by exhaustive search over all
codes with exact distances.
"""
from fractions import Fraction
import math
import struct

import numpy as np


def f32(x) -> float:
    """Round-trip a Python float through binary32 storage."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def frac_to_f32(r: Fraction) -> float:
    """Nearest binary32 to the exact rational r (ties to even), with subnormals;
    no overflow handling (callers stay in range)."""
    if r == 0:
        return 0.0
    sign = -1.0 if r < 0 else 1.0
    a = abs(r)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix possible off-by-one of the float log
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp_e = max(e, -126) - 23
    ulp = Fraction(2) ** ulp_e
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(fl * ulp)


def frac_to_bf16_bits(r: Fraction) -> int:
    """bf16 bit pattern of the nearest bf16 to the exact rational r (ties to
    even; 7 fraction bits, subnormal quantum 2^-133); r == 0 gives +0; no
    overflow handling (callers stay in range)."""
    if r == 0:
        return 0
    sign = 0x8000 if r < 0 else 0
    a = abs(r)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (max(e, -126) - 7)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = float(fl * ulp)  # a bf16 value, so exact in binary32 too
    return sign | (struct.unpack("<I", struct.pack("<f", val))[0] >> 16)


def bf16_all_positive_finite() -> np.ndarray:
    """All positive finite bf16 values as float32 (32,639 of them)."""
    bits = np.arange(1, 0x7F80, dtype=np.uint32)
    return (bits << 16).view(np.float32)


def nearest_e4m3_exhaustive(v: float, table) -> int:
    """E4M3FN code nearest to v by exhaustive search with exact distances;
    ties to the even code; |v| >= 448 saturates; the sign of zero is kept."""
    neg = math.copysign(1.0, v) < 0
    a = Fraction(abs(v))
    if a >= 448:
        best = 0x7E
    else:
        best, bestd = None, None
        for c in range(127):
            d = abs(Fraction(table[c]) - a)
            if bestd is None or d < bestd or (d == bestd and c % 2 == 0):
                best, bestd = c, d
    return best | (0x80 if neg else 0)
