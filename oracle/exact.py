"""Exact-arithmetic GEMM for tiny shapes, with Python fractions.

Test infrastructure only (see the package header).

Every E4M3 value and every fp32 scale is a dyadic rational, so the sum that
defines D can be formed exactly and rounded to bf16 exactly.  Used to check
the float64 oracle on brute-force cases; pure Python loops, tiny sizes only.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .e4m3 import decode_scalar


def _frac(v) -> Fraction:
    return Fraction(float(v))   # exact for finite binary floats


def gemm_nt_exact(a, sfa, b, sfb):
    """List-of-lists of Fractions: the exact D before rounding."""
    m, k = a.shape
    n = b.shape[0]
    dec_a = [[Fraction(decode_scalar(int(a[i, kk]))) for kk in range(k)] for i in range(m)]
    dec_b = [[Fraction(decode_scalar(int(b[j, kk]))) for kk in range(k)] for j in range(n)]
    out = []
    for i in range(m):
        row = []
        for j in range(n):
            total = Fraction(0)
            for kb in range(k // 128):
                part = sum(dec_a[i][kk] * dec_b[j][kk] for kk in range(kb * 128, (kb + 1) * 128))
                total += _frac(sfa[i, kb]) * _frac(sfb[j // 128, kb]) * part
            row.append(total)
        out.append(row)
    return out


def round_fraction_to_bf16_bits(x: Fraction) -> int:
    """Exact round-to-nearest-even of a rational to bf16 bits."""
    if x == 0:
        return 0
    neg = x < 0
    a = -x if neg else x
    # Leading-bit exponent e: 2^e <= a < 2^(e+1).
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = max(e, -126) - 7
    scaled = a / (Fraction(2) ** q)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = Fraction(n) * Fraction(2) ** q
    if v >= Fraction(2) ** 128:
        bits = 0x7F80
    else:
        bits = int(np.array([float(v)], dtype=np.float32).view(np.uint32)[0] >> 16)
    return bits | (0x8000 if neg else 0)


def is_bf16_tie(x: Fraction) -> bool:
    """True when x lies exactly halfway between two bf16 values."""
    if x == 0:
        return False
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = max(e, -126) - 7
    scaled = a / (Fraction(2) ** q)
    return scaled - (scaled.numerator // scaled.denominator) == Fraction(1, 2)
