"""Fine-grained FP8 quantizers: 1x128 per-token blocks and 128x128 weight blocks.

Test infrastructure only (see the package header).

What is quantized and at which granularity follows the method's block scaling:
one fp32 scale per row per 128-wide K block for activations and one per
128x128 block for weights (page "GitHub 推荐：…DeepGEMM…", 问题判断 on
128x128 block scaling; page juejin.cn, section 1 on fine-grained scaling).
The pages leave the arithmetic of a scale open; the readings taken:

1. amax = max |x| over the block (exact in fp32).
2. amax' = max(amax, fp32(1e-4)), so an all-zero block still has a positive scale.
3. s = fl32(amax' / 448)  (IEEE fp32 division, round to nearest even).
4. UE8M0 mode (exponent-only scales): s <- 2^ceil(log2 s), taken on the fp32
   bits: a scale with non-zero mantissa bits moves to the next power of two.
5. t = fl32(x / s) (IEEE fp32 division), clamped to [-448, 448], then encoded
   to E4M3 with ties to even.

A partial last block (rows of B beyond a multiple of 128) is quantized over
its real rows only.
"""
from __future__ import annotations

import numpy as np

from . import e4m3

BLOCK = 128
AMAX_FLOOR = np.float32(1e-4)
E4M3_MAX = np.float32(448.0)


def ue8m0_round_up(s: np.ndarray) -> np.ndarray:
    """Smallest power of two >= s, for positive normal fp32 s."""
    s = np.asarray(s, dtype=np.float32)
    bits = s.view(np.uint32)
    exp_bits = bits & np.uint32(0x7F800000)
    has_mant = (bits & np.uint32(0x007FFFFF)) != 0
    out = np.where(has_mant, exp_bits + np.uint32(0x00800000), exp_bits).astype(np.uint32)
    return out.view(np.float32)


def block_scale(amax: np.ndarray, ue8m0: bool) -> np.ndarray:
    """fp32 scale of a block from its fp32 amax (steps 2-4 above)."""
    amax = np.asarray(amax, dtype=np.float32)
    s = (np.maximum(amax, AMAX_FLOOR) / E4M3_MAX).astype(np.float32)
    return ue8m0_round_up(s) if ue8m0 else s


def encode_scaled(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Codes of fp32 ``x`` under fp32 scale ``s`` (broadcastable): step 5."""
    t = (np.asarray(x, dtype=np.float32) / np.asarray(s, dtype=np.float32)).astype(np.float32)
    t = np.clip(t, -E4M3_MAX, E4M3_MAX)
    return e4m3.encode(t)


def per_token_cast(x: np.ndarray, ue8m0: bool = False):
    """x fp32 (or bf16 widened exactly to fp32) [M, K], K % 128 == 0.

    Returns (codes uint8 [M, K], scales fp32 [M, K/128]).
    """
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 128")
    blocks = x.reshape(m, k // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=2)
    s = block_scale(amax, ue8m0)
    q = encode_scaled(blocks, s[:, :, None]).reshape(m, k)
    return q, s


def per_block_cast(w: np.ndarray, ue8m0: bool = False):
    """w fp32 [N, K], K % 128 == 0; 128x128 blocks, the last row block may be partial.

    Returns (codes uint8 [N, K], scales fp32 [ceil(N/128), K/128]).
    """
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 128")
    nb, kb = -(-n // BLOCK), k // BLOCK
    q = np.empty((n, k), dtype=np.uint8)
    s = np.empty((nb, kb), dtype=np.float32)
    for bi in range(nb):
        rows = w[bi * BLOCK:(bi + 1) * BLOCK]                      # real rows only
        blk = rows.reshape(rows.shape[0], kb, BLOCK)
        amax = np.abs(blk).max(axis=(0, 2))
        s[bi] = block_scale(amax, ue8m0)
        q[bi * BLOCK:(bi + 1) * BLOCK] = encode_scaled(blk, s[bi][None, :, None]).reshape(rows.shape[0], k)
    return q, s


def dequantize_rows(codes: np.ndarray, scales_per_kblock: np.ndarray) -> np.ndarray:
    """float64 dec(code) * scale, one scale per row per 128-wide K block.

    Exact: a decoded E4M3 value has at most 4 significant bits and an fp32
    scale 24, so their product fits the 53 bits of float64.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    r, k = codes.shape
    sc = np.repeat(np.asarray(scales_per_kblock, dtype=np.float64), BLOCK, axis=1)
    assert sc.shape == (r, k)
    return e4m3.decode(codes) * sc
