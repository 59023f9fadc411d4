"""Reference FP8 block-scaled GEMMs (dense, M-grouped contiguous, M-grouped masked).

Test infrastructure only (see the package header).

Definition (what every variant computes), D(bf16) = A . B^T with NT layout:

    D[i, j] = RNE_bf16( sum_kb  sa[i, kb] * sb[j // 128, kb] * sum_{k in kb} dec(A[i, k]) * dec(B[j, k]) )

* A: E4M3 [M, K] with one fp32 scale per row per 128-wide K block (sa);
  B: E4M3 [N, K] with one fp32 scale per 128x128 block (sb).  Block scaling
  and its granularity: page "GitHub 推荐：…DeepGEMM…", 问题判断; NT layout
  (both operands K-major): page ssnai.com "DeepGEMM" analysis, the SM90 vs
  SM100 notes on memory layout.
* Each K block's partial product is scaled and promoted into a higher-precision
  accumulator (two-level accumulation: page juejin.cn, sections 3 and 4(1);
  page "GitHub 推荐…", 创新之处 on per-block scaling through CUDA-core
  promotion).  The oracle gets the same real number without any blocking:
  dec(A)*sa and dec(B)*sb are exact in float64, their product is summed in
  float64 by a library matmul (any order; error ~K*2^-53 relative to the sum
  of magnitudes) and rounded once to bf16, round-to-nearest-even.
* Grouping is along M only; N and K are shared by all groups (page juejin.cn,
  section 3, grouped GEMM).  Contiguous layout: rows of all experts are
  concatenated and each expert segment is aligned to the M block; masked
  layout: per-group padded rows of which only the first masked_m[g] are valid
  (page juejin.cn, section 4(3)).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .bf16 import bf16_bits_to_float64, round_to_bf16_bits
from .quant import BLOCK, dequantize_rows


def _b_row_scales(sfb: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """[len(rows), K/128] scale of each B row: its 128-row block's scales."""
    return np.asarray(sfb, dtype=np.float64)[np.asarray(rows) // BLOCK]


def gemm_nt_fp64(a: np.ndarray, sfa: np.ndarray, b: np.ndarray, sfb: np.ndarray) -> np.ndarray:
    """float64 sum (before bf16 rounding) of the dense problem."""
    a64 = dequantize_rows(a, sfa)
    b64 = dequantize_rows(b, _b_row_scales(sfb, np.arange(b.shape[0])))
    return a64 @ b64.T


def gemm_nt(a: np.ndarray, sfa: np.ndarray, b: np.ndarray, sfb: np.ndarray,
            c: Optional[np.ndarray] = None) -> np.ndarray:
    """Dense reference: bf16 bits uint16 [M, N].

    With ``c`` (fp32 [M, N]): D = RNE_bf16(C + A . B^T), the accumulating form of
    the call (page "GitHub 推荐…DeepGEMM…", 解法哲学: the optional ``c`` argument
    of fp8_gemm_nt; the pages give no more, and the reading taken is an fp32
    addend of D's shape, added exactly before the single rounding).
    """
    acc = gemm_nt_fp64(a, sfa, b, sfb)
    if c is not None:
        acc = acc + np.asarray(c, dtype=np.float32).astype(np.float64)
    return round_to_bf16_bits(acc)


def gemm_nt_sampled(a: np.ndarray, sfa: np.ndarray, b: np.ndarray, sfb: np.ndarray,
                    rows: Sequence[int], cols: Sequence[int]) -> np.ndarray:
    """D[rows][:, cols] of the dense problem, decoding only the rows it needs."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    a64 = dequantize_rows(a[rows], sfa[rows])
    b64 = dequantize_rows(b[cols], _b_row_scales(sfb, cols))
    return round_to_bf16_bits(a64 @ b64.T)


def gemm_nt_columns(a_rows: np.ndarray, sfa_rows: np.ndarray, b_rows: np.ndarray,
                    sfb_rows: np.ndarray) -> np.ndarray:
    """D for some rows of A and some output columns, given directly.

    a_rows [R, K] with sfa_rows [R, K/128]; b_rows [C, K] are the B rows of the
    wanted output columns and sfb_rows [C, K/128] the scales of the 128-row
    block each of them belongs to.  Returns bf16 bits [R, C].
    """
    a64 = dequantize_rows(a_rows, sfa_rows)
    b64 = dequantize_rows(b_rows, sfb_rows)
    return round_to_bf16_bits(a64 @ b64.T)


def m_grouped_contiguous(a: np.ndarray, sfa: np.ndarray, b: np.ndarray, sfb: np.ndarray,
                         m_indices: np.ndarray, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Row i with g = m_indices[i] >= 0 gets the dense result against B[g];
    rows with -1 keep what ``out`` holds (they are not part of the result).

    a [M_total, K], sfa [M_total, K/128], b [G, N, K], sfb [G, ceil(N/128), K/128].
    """
    m_total = a.shape[0]
    n = b.shape[1]
    d = np.zeros((m_total, n), np.uint16) if out is None else out.copy()
    m_indices = np.asarray(m_indices)
    for g in range(b.shape[0]):
        rows = np.nonzero(m_indices == g)[0]
        if rows.size:
            d[rows] = gemm_nt(a[rows], sfa[rows], b[g], sfb[g])
    return d


def m_grouped_masked(a: np.ndarray, sfa: np.ndarray, b: np.ndarray, sfb: np.ndarray,
                     masked_m: np.ndarray, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Group g, row i < masked_m[g] gets the dense result of A[g, i] against B[g];
    rows at or beyond masked_m[g] keep what ``out`` holds.

    a [G, max_m, K], sfa [G, max_m, K/128], b [G, N, K], sfb [G, ceil(N/128), K/128].
    masked_m values beyond max_m count as max_m.
    """
    num_groups, max_m, _ = a.shape
    n = b.shape[1]
    d = np.zeros((num_groups, max_m, n), np.uint16) if out is None else out.copy()
    for g in range(num_groups):
        mm = int(min(max(int(masked_m[g]), 0), max_m))
        if mm:
            d[g, :mm] = gemm_nt(a[g, :mm], sfa[g, :mm], b[g], sfb[g])
    return d


def as_float(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_float64(bits)
