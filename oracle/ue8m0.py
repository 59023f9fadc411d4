"""Packed UE8M0 scale words: exponent-only scales, four per int32.

Test infrastructure only (see the package header).

Format (page "GitHub 推荐：DeepSeek 开源周最大黑马 DeepGEMM…", 可复用的模式与技巧,
"UE8M0 int32 packing"; page ssnai.com DeepGEMM analysis, on the scale formats):
an unsigned 8-bit exponent e stands for the scale 2^(e - 127); four of them,
for four consecutive 128-wide K blocks, share one 32-bit word, the first block
in the least significant byte.  The pages give no formula for turning an fp32
scale into an exponent; the reading taken is the smallest power of two that is
>= the scale (the same rounding the quantizer's UE8M0 mode uses), which is the
exact exponent for a scale that already is a power of two.  Bytes past the last
K block are 0.
"""
from __future__ import annotations

import math

import numpy as np


def exponent_of(s: float) -> int:
    """UE8M0 exponent of one positive normal fp32 scale: 127 + ceil(log2 s).

    Written from frexp (s = f * 2^x with f in [0.5, 1)): log2 s lies in
    [x - 1, x), so ceil(log2 s) = x unless f == 0.5 exactly (s = 2^(x-1)).
    """
    f, x = math.frexp(float(np.float32(s)))
    return 127 + (x - 1 if f == 0.5 else x)


def pack(sf: np.ndarray) -> np.ndarray:
    """fp32 scales [rows, kblocks] -> int32 words [rows, ceil(kblocks / 4)]."""
    sf = np.asarray(sf, dtype=np.float32)
    rows, kblocks = sf.shape
    words = (kblocks + 3) // 4
    out = np.zeros((rows, words), dtype=np.uint32)
    for i in range(rows):
        for kb in range(kblocks):
            e = exponent_of(sf[i, kb])
            out[i, kb // 4] |= np.uint32(e) << np.uint32(8 * (kb % 4))
    return out.view(np.int32)


def unpack(words: np.ndarray, kblocks: int) -> np.ndarray:
    """int32 words [rows, ceil(kblocks / 4)] -> fp32 scales 2^(e - 127) [rows, kblocks]."""
    w = np.asarray(words, dtype=np.int32).view(np.uint32)
    rows = w.shape[0]
    out = np.empty((rows, kblocks), dtype=np.float32)
    for i in range(rows):
        for kb in range(kblocks):
            e = int((w[i, kb // 4] >> np.uint32(8 * (kb % 4))) & np.uint32(0xFF))
            out[i, kb] = np.float32(math.ldexp(1.0, e - 127))
    return out
