"""OCP E4M3 ("FN" flavour) decode and round-to-nearest-even encode, on the CPU.

Test infrastructure only (see the package header).

The format: the pages fix it as 4 exponent bits and 3 mantissa bits, used for
GEMM inputs (page "企业官网建设流程全解析", section 2.3 on FP8 formats); the
workload text adds the OCP flavour with largest finite magnitude 448.  Field
layout (OCP 8-bit floating point, E4M3):

* sign s (bit 7), exponent e (bits 6..3, bias 7), mantissa m (bits 2..0);
* e >= 1: (-1)^s * 2^(e-7) * (1 + m/8);  e == 0: (-1)^s * 2^-6 * (m/8);
* S.1111.111 is NaN; there is no infinity; the largest finite value is 448.
"""
from __future__ import annotations

import numpy as np

NAN_CODES = (0x7F, 0xFF)
MAX_FINITE = 448.0


def decode_scalar(code: int) -> float:
    """Value of one code, straight from the field definition."""
    code = int(code) & 0xFF
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    sign = -1.0 if s else 1.0
    if e == 0:
        return sign * 2.0 ** -6 * (m / 8.0)
    return sign * 2.0 ** (e - 7) * (1.0 + m / 8.0)


# Decode table for all 256 codes (float64; every finite value is exact).
DECODE_TABLE = np.array([decode_scalar(c) for c in range(256)], dtype=np.float64)


def decode(codes: np.ndarray) -> np.ndarray:
    """float64 values of an array of uint8 codes."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


# Non-negative finite codes 0x00..0x7E in increasing value order (code == index).
_POS_VALUES = DECODE_TABLE[:0x7F]
assert np.all(np.diff(_POS_VALUES) > 0)


def encode(t: np.ndarray) -> np.ndarray:
    """Codes of finite values already clamped to [-448, 448].

    Round to nearest; when a value lies exactly halfway between two adjacent
    representable magnitudes, pick the one whose mantissa LSB is 0 ("ties to
    even").  Normals and subnormals alike, no flush to zero.  The sign bit is
    always copied from the input, so -0 and tiny negatives give 0x80.
    """
    t = np.asarray(t, dtype=np.float64)
    if np.any(~np.isfinite(t)) or np.any(np.abs(t) > MAX_FINITE):
        raise ValueError("encode expects finite values within [-448, 448]")
    neg = np.signbit(t)
    a = np.abs(t)
    # Neighbours lo <= a <= hi among representable magnitudes.
    hi = np.searchsorted(_POS_VALUES, a, side="left")          # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.where(_POS_VALUES[hi] == a, hi, np.maximum(hi - 1, 0))
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | (neg.astype(np.uint8) << 7)
