"""Pins of the packed UE8M0 scale oracle (oracle/ue8m0.py), CPU only.

* A hand-worked word: exponents 127, 128, 126, 130 (scales 1, 2, 1/2, 8) in
  bytes 0..3 make 0x827E807F.
* Rounding up: the exponent from frexp agrees with the quantizer's bit-level
  UE8M0 rounding (an independent formulation) on random and edge scales.
* Every exponent 1..254 unpacks to the exact power of two, and packing then
  unpacking power-of-two scales is the identity.
* Bytes past the last K block are zero; the byte order is little-endian.
"""
import numpy as np
import pytest

from oracle import quant, ue8m0


def test_hand_worked_word():
    w = ue8m0.pack(np.array([[1.0, 2.0, 0.5, 8.0]], dtype=np.float32))
    assert w.shape == (1, 1)
    assert int(w.view(np.uint32)[0, 0]) == 0x827E807F
    assert np.array_equal(ue8m0.unpack(w, 4), np.array([[1.0, 2.0, 0.5, 8.0]], dtype=np.float32))


@pytest.mark.parametrize("s,e", [(1.0, 127), (0.75, 127), (0.5, 126), (0.5000001, 127), (3.0, 129),
                                 (2.0 ** -20, 107), (448.0 / 448.0, 127), (1e-4 / 448, 105)])
def test_exponent_examples(s, e):
    assert ue8m0.exponent_of(np.float32(s)) == e


def test_exponent_matches_bit_level_round_up():
    rng = np.random.default_rng(0)
    s = np.concatenate([
        (2.0 ** rng.uniform(-60, 60, 4000)).astype(np.float32),
        np.float32(2.0) ** np.arange(-100, 100, dtype=np.float32),
        np.nextafter(np.float32(2.0) ** np.arange(-100, 100, dtype=np.float32), np.float32(np.inf)),
        np.nextafter(np.float32(2.0) ** np.arange(-100, 100, dtype=np.float32), np.float32(0)),
    ]).astype(np.float32)
    bits_e = ((quant.ue8m0_round_up(s).view(np.uint32) >> 23) & 0xFF).astype(int)
    mine = np.array([ue8m0.exponent_of(x) for x in s])
    assert np.array_equal(mine, bits_e)


def test_every_exponent_unpacks_exactly():
    e = np.arange(1, 255, dtype=np.uint32)
    pad = (-len(e)) % 4
    e = np.concatenate([e, np.full(pad, 127, np.uint32)])
    words = (e[0::4] | (e[1::4] << 8) | (e[2::4] << 16) | (e[3::4] << 24)).astype(np.uint32)
    got = ue8m0.unpack(words.view(np.int32)[None, :], len(e))[0]
    want = np.array([2.0 ** (int(x) - 127) for x in e], dtype=np.float64)
    assert np.array_equal(got.astype(np.float64), want)


def test_roundtrip_and_padding():
    rng = np.random.default_rng(1)
    for kblocks in (1, 2, 3, 4, 5, 7, 9):
        sf = (np.float32(2.0) ** rng.integers(-30, 10, size=(6, kblocks)).astype(np.float32)).astype(np.float32)
        w = ue8m0.pack(sf)
        assert w.shape == (6, (kblocks + 3) // 4)
        assert np.array_equal(ue8m0.unpack(w, kblocks), sf)
        last = w.view(np.uint32)[:, -1]
        used = kblocks - 4 * (w.shape[1] - 1)
        if used < 4:
            assert np.all((last >> np.uint32(8 * used)) == 0)
