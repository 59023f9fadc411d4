"""Round float64 values to bfloat16, round-to-nearest-even, in one step.

Test infrastructure only (see the package header).

The GEMM output is bf16 (the API names of the pages end in ``_bf16_nt``, page
juejin.cn "DeepGEMM 简介…", section 5).  The oracle rounds its float64 sum
directly to bf16; going through fp32 first could round twice.

bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 stored mantissa bits; the
significand has 8 bits; normals down to 2^-126, subnormals in steps of 2^-133;
magnitudes that round past the largest finite value become infinity.
"""
from __future__ import annotations

import numpy as np


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns of float64 ``x`` (RNE, overflow -> +-inf)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)):
        raise ValueError("NaN input")
    neg = np.signbit(x)
    a = np.abs(x)
    out = np.zeros(a.shape, dtype=np.float64)
    nz = (a != 0) & np.isfinite(a)
    _, ex = np.frexp(a[nz])                    # a = f * 2^ex, f in [0.5, 1)
    lead = ex.astype(np.int64) - 1             # exponent of the leading bit
    q_exp = np.maximum(lead, -126) - 7         # spacing of bf16 values there
    n = np.rint(np.ldexp(a[nz], -q_exp))       # exact scaling; rint is ties-to-even
    out[nz] = np.ldexp(n, q_exp)
    out[np.isinf(a)] = np.inf
    out[out >= 2.0 ** 128] = np.inf
    f32 = out.astype(np.float32)               # exact: <= 8 significant bits
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    return bits | (neg.astype(np.uint16) << 15)


def bf16_bits_to_float64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
