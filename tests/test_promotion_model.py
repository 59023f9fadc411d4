"""Why the method promotes each K block into fp32 (two-level accumulation).

The pages (juejin.cn post, section 3) report that the FP8 tensor-core path
accumulates with only about 14 bits, which costs about 2% of relative error on
two random K = 4096 matrices, and that promoting every 128-wide K block into
an fp32 accumulator fixes it.  This models that on the CPU: products of
quantized operands (exact in float64) summed by an accumulator that keeps 14
significant bits and truncates after every addition, once over all of K and
once per 128-wide block with the blocks' sums added in fp32.  The model is an
assumption (the pages do not say how the narrow accumulator rounds), so the
check is qualitative: a percent-level error without promotion, at least ten
times less with it.  The kernels' own accumulation is pinned bit for bit
elsewhere (the GPU accumulator-width tests).
"""
import numpy as np

from oracle import quant


def _narrow(x, bits=14):
    m, e = np.frexp(x)                  # x = m * 2^e, 0.5 <= |m| < 1
    s = 2.0 ** bits
    return np.trunc(m * s) / s * 2.0 ** e


def test_block_promotion_bounds_the_narrow_accumulator_error():
    rng = np.random.default_rng(5)
    m = n = 64
    k = 4096
    a = rng.standard_normal((m, k)).astype(np.float32)
    b = rng.standard_normal((n, k)).astype(np.float32)
    qa, sa = quant.per_token_cast(a)
    qb, sb = quant.per_block_cast(b)
    a64 = quant.dequantize_rows(qa, sa)
    b64 = quant.dequantize_rows(qb, np.asarray(sb, np.float64)[np.arange(n) // 128])
    exact = a64 @ b64.T
    prod = a64[:, None, :] * b64[None, :, :]          # exact products, float64
    flat = np.zeros((m, n))
    for kk in range(k):
        flat = _narrow(flat + prod[:, :, kk])
    promoted = np.zeros((m, n), dtype=np.float32)
    for kb in range(k // 128):
        part = np.zeros((m, n))
        for kk in range(kb * 128, (kb + 1) * 128):
            part = _narrow(part + prod[:, :, kk])
        promoted += part.astype(np.float32)
    scale = np.abs(exact).max()
    err_flat = np.abs(flat - exact).max() / scale
    err_promoted = np.abs(promoted.astype(np.float64) - exact).max() / scale
    assert err_flat > 1e-2, err_flat
    assert err_promoted < err_flat / 10, (err_promoted, err_flat)
