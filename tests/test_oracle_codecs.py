"""Pins of the oracle's E4M3 codec and bf16 rounding against things other than itself:
torch's CPU float8_e4m3fn / bfloat16 conversions (library routines), hand-derived
golden values, an independent closed-form encoder and hand-picked tie cases."""
import os

import numpy as np
import pytest
import torch

from oracle import bf16, e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_decode_all():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().double().numpy()


def test_decode_matches_torch_for_all_codes():
    ref = _torch_decode_all()
    ours = e4m3.DECODE_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    # signs of zeros
    assert not np.signbit(ours[0x00]) and np.signbit(ours[0x80])


def test_decode_golden_table():
    for line in open(os.path.join(GOLDEN, "e4m3_values.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, value = line.split()[:2]
        got = e4m3.DECODE_TABLE[int(code, 16)]
        if value == "nan":
            assert np.isnan(got)
        else:
            assert got == float(value) and np.signbit(got) == value.startswith("-"), code


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in e4m3.NAN_CODES], dtype=np.uint8)
    assert np.array_equal(e4m3.encode(e4m3.decode(codes)), codes)


def _closed_form_encode(t):
    """Second, independent formulation: scale by the local spacing, rint (ties to
    even), rebuild the bit fields."""
    t = np.asarray(t, np.float64)
    neg = np.signbit(t)
    a = np.abs(t)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    lead = np.where(a > 0, ex - 1, -6)
    q = np.maximum(lead, -6) - 3                # 4 significant bits; subnormal spacing 2^-9
    n = np.rint(np.ldexp(a, -q)).astype(np.int64)
    lead2 = np.where(n >= 16, lead + 1, lead)   # carry into the next binade
    n = np.where(n >= 16, n // 2, n)
    sub = (lead2 < -6) | (n < 8)
    e_field = np.where(sub, 0, lead2 + 7)
    m_field = np.where(sub, n, n - 8)
    return ((neg.astype(np.int64) << 7) | (e_field << 3) | m_field).astype(np.uint8)


def test_encode_ties_to_even_at_every_midpoint():
    pos = e4m3.DECODE_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2               # exact in float64
    got = e4m3.encode(mids)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(got, expect)
    assert np.array_equal(e4m3.encode(-mids), expect | 0x80)
    # just off the midpoint, nearest wins
    above = np.nextafter(mids.astype(np.float32), np.float32(1e9)).astype(np.float64)
    below = np.nextafter(mids.astype(np.float32), np.float32(-1e9)).astype(np.float64)
    assert np.array_equal(e4m3.encode(above), (lo + 1).astype(np.uint8))
    assert np.array_equal(e4m3.encode(below), lo.astype(np.uint8))


def test_encode_keeps_sign_of_zero_and_tiny_negatives():
    got = e4m3.encode(np.array([0.0, -0.0, -1e-30, 1e-30, -2.0 ** -11, 2.0 ** -10 * 1.5]))
    assert got.tolist() == [0x00, 0x80, 0x80, 0x00, 0x80, 0x01]


@pytest.mark.slow
def test_encode_sweep_matches_torch_and_closed_form():
    # Every 37th fp32 bit pattern in [0, 448], plus its negation: ~29M values.
    top = int(np.float32(448.0).view(np.uint32))
    bits = np.arange(0, top + 1, 37, dtype=np.uint32)
    bits = np.concatenate([bits, np.array([top], np.uint32)])
    t32 = bits.view(np.float32)
    for sign in (1.0, -1.0):
        t = (t32 * np.float32(sign)).astype(np.float32)
        ours = e4m3.encode(t.astype(np.float64))
        ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(ours, ref)
        assert np.array_equal(ours, _closed_form_encode(t))


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        e4m3.encode(np.array([449.0]))
    with pytest.raises(ValueError):
        e4m3.encode(np.array([np.nan]))


# ------------------------------------------------------------------ bf16

def _torch_bf16_bits(x32):
    return torch.from_numpy(np.asarray(x32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # keep away from the overflow edge, handled separately
    x = x[np.abs(x) < np.float32(3.0e38)]
    assert np.array_equal(bf16.round_to_bf16_bits(x.astype(np.float64)), _torch_bf16_bits(x))


def test_bf16_hand_picked_cases():
    cases = [
        (1.0, 0x3F80),
        (1.0 + 2.0 ** -8, 0x3F80),                   # tie -> even (down)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),               # tie -> even (up)
        (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),      # above the tie: up.  Via fp32 it would tie and go down
        (-2.5, 0xC020),
        (2.0 ** -133, 0x0001),                       # smallest subnormal
        (2.0 ** -134, 0x0000),                       # tie between 0 and 2^-133 -> 0
        (3 * 2.0 ** -134, 0x0002),                   # tie between 1 and 2 (x 2^-133) -> 2
        (2.0 ** -126, 0x0080),                       # smallest normal
        ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),      # largest finite
        (2.0 ** 128 - 2.0 ** 119, 0x7F80),           # tie at the top -> infinity
        (2.0 ** 128 - 2.0 ** 119 - 2.0 ** 100, 0x7F7F),
        (-1e300, 0xFF80),
        (0.0, 0x0000),
        (-0.0, 0x8000),
    ]
    xs = np.array([c[0] for c in cases], dtype=np.float64)
    got = bf16.round_to_bf16_bits(xs)
    assert got.tolist() == [c[1] for c in cases]


def test_bf16_roundtrip_float():
    bits = np.arange(0, 0x7F80, 3, dtype=np.uint16)
    assert np.array_equal(bf16.round_to_bf16_bits(bf16.bf16_bits_to_float64(bits)), bits)
