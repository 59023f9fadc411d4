"""Pins of the oracle GEMMs: exact rational brute force, reductions to integer
matmuls and closed forms, and the invariants the definition implies.

Each check targets a plausible mistake: a transposed operand or swapped scale
index (identity and distinct per-block scales), a dropped K block (single-block
case), a wrong rounding (int64 sums against torch's fp32->bf16), a group mix-up
(independence, grouped == dense)."""
import numpy as np
import pytest
import torch

from oracle import bf16, e4m3, exact, gemm, quant

FINITE = np.array([c for c in range(256) if c not in e4m3.NAN_CODES], dtype=np.uint8)


def _random_codes(rng, shape, special=True):
    c = rng.choice(FINITE, size=shape)
    if special:  # sprinkle subnormals, +-448 and signed zeros
        flat = c.reshape(-1)
        idx = rng.integers(0, flat.size, size=max(1, flat.size // 8))
        flat[idx] = rng.choice(np.array([0x00, 0x80, 0x01, 0x81, 0x07, 0x7E, 0xFE], np.uint8), size=idx.size)
    return c


def _random_scales(rng, shape, pow2):
    if pow2:
        return np.exp2(rng.integers(-10, 10, size=shape)).astype(np.float32)
    return (np.exp2(rng.uniform(-10, 10, size=shape))).astype(np.float32)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_matches_exact_rationals(seed):
    rng = np.random.default_rng(100 + seed)
    m, n = int(rng.integers(1, 9)), int(rng.integers(1, 9))
    k = int(rng.choice([128, 256, 384]))
    pow2 = bool(seed % 2)
    a = _random_codes(rng, (m, k))
    b = _random_codes(rng, (n, k))
    sfa = _random_scales(rng, (m, k // 128), pow2)
    sfb = _random_scales(rng, (1, k // 128), pow2)
    got = gemm.gemm_nt(a, sfa, b, sfb)
    ex = exact.gemm_nt_exact(a, sfa, b, sfb)
    d64 = gemm.gemm_nt_fp64(a, sfa, b, sfb)
    from fractions import Fraction
    mismatches = 0
    for i in range(m):
        for j in range(n):
            want = exact.round_fraction_to_bf16_bits(ex[i][j])
            if int(got[i, j]) != want:
                # only allowed where float64 summation was inexact and the exact value is a tie
                assert Fraction(float(d64[i, j])) != ex[i][j] and exact.is_bf16_tie(ex[i][j])
                mismatches += 1
    assert mismatches == 0 or mismatches <= 1


def _int_codes(rng, shape, lo=-16, hi=16):
    vals = rng.integers(lo, hi + 1, size=shape).astype(np.float64)
    return e4m3.encode(vals), vals.astype(np.int64)


def test_unit_scales_reduce_to_int64_matmul_and_torch_rounding():
    rng = np.random.default_rng(21)
    m, n, k = 16, 200, 512                      # N not a multiple of 128
    a, ai = _int_codes(rng, (m, k))
    b, bi = _int_codes(rng, (n, k))
    sfa = np.ones((m, k // 128), np.float32)
    sfb = np.ones((2, k // 128), np.float32)
    got = gemm.gemm_nt(a, sfa, b, sfb)
    ref_int = ai @ bi.T                          # exact, |sum| < 2^24
    assert np.abs(ref_int).max() < 2 ** 24
    ref = torch.from_numpy(ref_int.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_identity_b_picks_the_right_scales():
    rng = np.random.default_rng(22)
    m, k = 8, 256
    n = k
    a = _random_codes(rng, (m, k), special=False)
    b = np.zeros((n, k), np.uint8)
    b[np.arange(n), np.arange(n)] = 0x38         # 1.0 on the diagonal
    sfa = _random_scales(rng, (m, 2), False)
    sfb = _random_scales(rng, (2, 2), False)     # distinct per (n-block, k-block)
    got = gemm.gemm_nt(a, sfa, b, sfb)
    for i in range(m):
        for j in range(n):
            val = e4m3.DECODE_TABLE[a[i, j]] * float(sfa[i, j // 128]) * float(sfb[j // 128, j // 128])
            from fractions import Fraction
            want = exact.round_fraction_to_bf16_bits(Fraction(val))   # product exact in float64
            assert int(got[i, j]) == want


def test_all_ones_gives_k():
    for k in (512, 1536, 2048, 7168, 16384):
        a = np.full((2, k), 0x38, np.uint8)
        b = np.full((3, k), 0x38, np.uint8)
        got = gemm.gemm_nt(a, np.ones((2, k // 128), np.float32), b, np.ones((1, k // 128), np.float32))
        assert np.all(bf16.bf16_bits_to_float64(got) == float(k))


def test_single_nonzero_k_block():
    rng = np.random.default_rng(23)
    m, n, k = 4, 5, 384
    a, ai = _int_codes(rng, (m, k), -8, 8)
    b, bi = _int_codes(rng, (n, k), -8, 8)
    a[:, :128] = 0
    a[:, 256:] = 0
    ai[:, :128] = 0
    ai[:, 256:] = 0
    sfa = _random_scales(rng, (m, 3), True)
    sfb = _random_scales(rng, (1, 3), True)
    got = gemm.gemm_nt(a, sfa, b, sfb)
    p = ai[:, 128:256] @ bi[:, 128:256].T
    want = p.astype(np.float64) * sfa[:, 1:2].astype(np.float64) * float(sfb[0, 1])
    ref = torch.from_numpy(want.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.abs(p).max() < 2 ** 24
    assert np.array_equal(got, ref)


def _problem(rng, m, n, k, pow2=False):
    a = _random_codes(rng, (m, k), special=False)
    b = _random_codes(rng, (n, k), special=False)
    return a, _random_scales(rng, (m, k // 128), pow2), b, _random_scales(rng, (-(-n // 128), k // 128), pow2)


def test_power_of_two_scale_linearity_is_bit_exact():
    rng = np.random.default_rng(24)
    a, sfa, b, sfb = _problem(rng, 8, 150, 256)
    base = bf16.bf16_bits_to_float64(gemm.gemm_nt(a, sfa, b, sfb))
    for p in (-3, 5):
        up_a = bf16.bf16_bits_to_float64(gemm.gemm_nt(a, sfa * np.float32(2.0 ** p), b, sfb))
        up_b = bf16.bf16_bits_to_float64(gemm.gemm_nt(a, sfa, b, sfb * np.float32(2.0 ** p)))
        assert np.array_equal(up_a, base * 2.0 ** p)
        assert np.array_equal(up_b, base * 2.0 ** p)


def test_negation_and_zero_rows():
    rng = np.random.default_rng(25)
    a, sfa, b, sfb = _problem(rng, 6, 40, 384)
    base = bf16.bf16_bits_to_float64(gemm.gemm_nt(a, sfa, b, sfb))
    neg = bf16.bf16_bits_to_float64(gemm.gemm_nt(a ^ np.uint8(0x80), sfa, b, sfb))
    assert np.array_equal(neg, -base)
    a2 = a.copy()
    a2[3] = 0
    z = bf16.bf16_bits_to_float64(gemm.gemm_nt(a2, sfa, b, sfb))
    assert np.all(z[3] == 0) and np.array_equal(np.delete(z, 3, 0), np.delete(base, 3, 0))


def test_sampled_matches_full():
    rng = np.random.default_rng(26)
    a, sfa, b, sfb = _problem(rng, 20, 300, 512)
    full = gemm.gemm_nt(a, sfa, b, sfb)
    rows, cols = [0, 7, 19], [1, 128, 255, 299]
    assert np.array_equal(gemm.gemm_nt_sampled(a, sfa, b, sfb, rows, cols), full[np.ix_(rows, cols)])


def test_columns_form_matches_full():
    rng = np.random.default_rng(29)
    a, sfa, b, sfb = _problem(rng, 9, 260, 384)
    full = gemm.gemm_nt(a, sfa, b, sfb)
    cols = np.array([0, 127, 128, 259])
    got = gemm.gemm_nt_columns(a[[2, 8]], sfa[[2, 8]], b[cols], sfb[cols // 128])
    assert np.array_equal(got, full[np.ix_([2, 8], cols)])


def test_contiguous_rows_follow_their_group_and_padding_is_untouched():
    rng = np.random.default_rng(27)
    g, n, k = 3, 64, 256
    m_indices = np.array([0] * 100 + [-1] * 28 + [2] * 128 + [1] * 5 + [-1] * 123, np.int32)
    mt = m_indices.size
    a = _random_codes(rng, (mt, k), special=False)
    sfa = _random_scales(rng, (mt, 2), False)
    b = _random_codes(rng, (g, n, k), special=False)
    sfb = _random_scales(rng, (g, 1, 2), False)
    sentinel = np.full((mt, n), 0x7FC1, np.uint16)
    d = gemm.m_grouped_contiguous(a, sfa, b, sfb, m_indices, out=sentinel)
    assert np.all(d[m_indices < 0] == 0x7FC1)
    for gg in range(g):
        rows = np.nonzero(m_indices == gg)[0]
        assert np.array_equal(d[rows], gemm.gemm_nt(a[rows], sfa[rows], b[gg], sfb[gg]))
    # changing another group's B leaves group 0 unchanged
    b2 = b.copy()
    b2[1] ^= 0x80
    d2 = gemm.m_grouped_contiguous(a, sfa, b2, sfb, m_indices, out=sentinel)
    assert np.array_equal(d2[m_indices == 0], d[m_indices == 0])
    assert not np.array_equal(d2[m_indices == 1], d[m_indices == 1])


def test_masked_rows_beyond_count_untouched_and_clamped():
    rng = np.random.default_rng(28)
    g, max_m, n, k = 4, 16, 32, 128
    a = _random_codes(rng, (g, max_m, k), special=False)
    sfa = _random_scales(rng, (g, max_m, 1), False)
    b = _random_codes(rng, (g, n, k), special=False)
    sfb = _random_scales(rng, (g, 1, 1), False)
    masked_m = np.array([0, 5, 16, 99], np.int32)          # 99 clamps to max_m
    sentinel = np.full((g, max_m, n), 0x1234, np.uint16)
    d = gemm.m_grouped_masked(a, sfa, b, sfb, masked_m, out=sentinel)
    assert np.all(d[0] == 0x1234)
    assert np.all(d[1, 5:] == 0x1234)
    for gg, mm in ((1, 5), (2, 16), (3, 16)):
        assert np.array_equal(d[gg, :mm], gemm.gemm_nt(a[gg, :mm], sfa[gg, :mm], b[gg], sfb[gg]))


def test_quantize_then_gemm_close_to_fp32_matmul():
    # end-to-end sanity of the whole oracle on the dense workload recipe
    import synth
    w = synth.config0()
    qa, sa = quant.per_token_cast(w.a)
    qb, sb = quant.per_block_cast(w.b)
    d = bf16.bf16_bits_to_float64(gemm.gemm_nt(qa, sa, qb, sb))
    ref = w.a.astype(np.float64) @ w.b.astype(np.float64).T
    rel = np.linalg.norm(d - ref) / np.linalg.norm(ref)
    assert rel < 0.05


@pytest.mark.parametrize("seed", range(4))
def test_accumulate_form_matches_exact_rationals(seed):
    # D = RNE_bf16(C + A.B^T): the fp32 addend enters the exact sum before the one rounding.
    from fractions import Fraction
    rng = np.random.default_rng(300 + seed)
    m, n, k = int(rng.integers(1, 7)), int(rng.integers(1, 7)), 256
    a, b = _random_codes(rng, (m, k)), _random_codes(rng, (n, k))
    sfa, sfb = _random_scales(rng, (m, 2), bool(seed % 2)), _random_scales(rng, (1, 2), bool(seed % 2))
    c = (rng.standard_normal((m, n)) * 1e4).astype(np.float32)
    got = gemm.gemm_nt(a, sfa, b, sfb, c)
    ex = exact.gemm_nt_exact(a, sfa, b, sfb)
    for i in range(m):
        for j in range(n):
            total = ex[i][j] + Fraction(float(c[i, j]))
            if not exact.is_bf16_tie(total):
                assert int(got[i, j]) == exact.round_fraction_to_bf16_bits(total)


def test_accumulate_special_cases():
    rng = np.random.default_rng(7)
    a, b = _random_codes(rng, (5, 384)), _random_codes(rng, (6, 384))
    sfa, sfb = _random_scales(rng, (5, 3), False), _random_scales(rng, (1, 3), False)
    assert np.array_equal(gemm.gemm_nt(a, sfa, b, sfb, np.zeros((5, 6), np.float32)), gemm.gemm_nt(a, sfa, b, sfb))
    c = rng.standard_normal((5, 6)).astype(np.float32)
    zero_a = np.zeros_like(a)
    want = torch.from_numpy(c).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gemm.gemm_nt(zero_a, sfa, b, sfb, c), want)   # library fp32 -> bf16 RNE
