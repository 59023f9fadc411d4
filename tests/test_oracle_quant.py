"""Pins of the oracle quantizers: hand-worked golden examples, exact-rational
division cases, closed forms, the partial last weight block, and the error
bound of the encoding."""
import os

import numpy as np

from oracle import e4m3, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines():
    for line in open(os.path.join(GOLDEN, "quant_examples.txt")):
        line = line.split("#")[0].strip()
        if line:
            yield [f.strip() for f in line.split("|")]


def test_golden_quant_examples():
    n = 0
    for name, ue, xs, scale, codes in _golden_lines():
        vals = [float(v) for v in xs.split()]
        x = np.zeros((1, 128), np.float32)
        x[0, :len(vals)] = vals
        q, s = quant.per_token_cast(x, ue8m0=bool(int(ue)))
        assert s.shape == (1, 1)
        assert abs(float(s[0, 0]) - float(scale)) <= 1e-7 * float(scale), name
        expect = [int(c, 16) for c in codes.split()]
        assert q[0, :len(expect)].tolist() == expect, name
        n += 1
    assert n == 6


def _division_cases():
    """Cases of tests/golden/quant_division_cases.txt (written in exact rational
    arithmetic by make_quant_division_cases.py): values and scale as fp32 bits."""
    for line in open(os.path.join(GOLDEN, "quant_division_cases.txt")):
        line = line.split("#")[0].strip()
        if line:
            name, ue, xs, scale, codes = [f.strip() for f in line.split("|")]
            vals = np.array([int(v, 16) for v in xs.split()], np.uint32).view(np.float32)
            yield name, bool(int(ue)), vals, np.uint32(int(scale, 16)), [int(c, 16) for c in codes.split()]


def test_division_cases_bit_exact():
    """The scale is the correctly rounded fp32 amax/448 and each code comes from
    the correctly rounded fp32 quotient x/s; a reciprocal multiply (amax*RN(1/448)
    or x*RN(1/s)) or a quotient rounded straight to E4M3 fails these cases."""
    n = 0
    for name, ue, vals, scale_bits, want in _division_cases():
        x = np.zeros((1, 128), np.float32)
        x[0, :vals.size] = vals
        q, s = quant.per_token_cast(x, ue8m0=ue)
        assert s.view(np.uint32)[0, 0] == scale_bits, name
        assert q[0, :vals.size].tolist() == want, name
        # the same block as the first row of a 128x128 weight block
        w = np.zeros((128, 128), np.float32)
        w[0] = x[0]
        qw, sw = quant.per_block_cast(w, ue8m0=ue)
        assert sw.view(np.uint32)[0, 0] == scale_bits, name
        assert qw[0, :vals.size].tolist() == want, name
        n += 1
    assert n == 20


def test_scale_closed_forms():
    assert quant.block_scale(np.float32(448.0), False) == np.float32(1.0)
    assert quant.block_scale(np.float32(7.0), False) == np.float32(2.0 ** -6)
    assert quant.block_scale(np.float32(896.0), False) == np.float32(2.0)
    # power-of-two rounding of the scale itself
    up = quant.ue8m0_round_up(np.array([0.75, 1.0, 1.0 + 2.0 ** -23, 2.0 ** -20 * 1.5, 3.0], np.float32))
    assert up.tolist() == [1.0, 1.0, 2.0, 2.0 ** -19, 4.0]
    # zero block: floor at fp32(1e-4)
    s0 = quant.block_scale(np.float32(0.0), False)
    assert s0 == np.float32(np.float32(1e-4) / np.float32(448.0))


def test_per_token_cast_identity_when_values_representable():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7F, size=(4, 256)).astype(np.uint8)
    codes[:, 0] = 0x7E        # every block holds +448 -> scale 1
    codes[:, 128] = 0x7E
    x = e4m3.decode(codes).astype(np.float32)
    q, s = quant.per_token_cast(x)
    assert np.all(s == 1.0)
    assert np.array_equal(q, codes)


def test_per_token_cast_error_bound():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 512)) * np.exp2(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    for ue in (False, True):
        q, s = quant.per_token_cast(x, ue8m0=ue)
        recon = e4m3.decode(q) * np.repeat(s.astype(np.float64), 128, axis=1)
        err = np.abs(recon - x)
        sc = np.repeat(s.astype(np.float64), 128, axis=1)
        # normal range: half a mantissa step (2^-4 relative); subnormal: half of 2^-9 * s.
        bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * sc) * (1 + 1e-6)
        assert np.all(err <= bound)
        # the largest element of each block maps to +-448 exactly (non-ue8m0) or within range
        amax_codes = np.abs(e4m3.decode(q)).reshape(64, -1, 128).max(axis=2)
        if not ue:
            assert np.all(amax_codes == 448.0)
        else:
            assert np.all((amax_codes >= 224.0) & (amax_codes <= 448.0))
        # ue8m0 scales are powers of two
        if ue:
            m, e = np.frexp(s)
            assert np.all(m == 0.5)


def test_per_block_cast_partial_last_block():
    rng = np.random.default_rng(5)
    w = rng.standard_normal((130, 256)).astype(np.float32)
    w[:128] *= 100.0                            # first row block much larger
    q, s = quant.per_block_cast(w)
    assert q.shape == (130, 256) and s.shape == (2, 2)
    # second block: only its 2 real rows set the scale
    for kb in range(2):
        amax = np.abs(w[128:, kb * 128:(kb + 1) * 128]).max()
        assert s[1, kb] == np.float32(amax / np.float32(448.0))
        amax0 = np.abs(w[:128, kb * 128:(kb + 1) * 128]).max()
        assert s[0, kb] == np.float32(amax0 / np.float32(448.0))
