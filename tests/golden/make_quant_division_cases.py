"""Writes quant_division_cases.txt: 1x128 quantization cases whose expected scale
and codes are derived here in exact rational arithmetic (``fractions``), with no
call into the oracle or the GPU library.

    python tests/golden/make_quant_division_cases.py

The rule being pinned (one fixed reading, since the pages leave the arithmetic
of a scale open): s = RN32(max(amax, 1e-4) / 448) and t = RN32(x / s), both
correctly rounded fp32 divisions, then t is clamped to +-448 and rounded to the
nearest E4M3 value, ties to the even code.  The cases are chosen where a
plausible variant of that rule gives a different answer:

* ``scale_div``   amax / 448 and amax * RN32(1/448) round to different fp32 scales;
* ``quot_div``    x / s and x * RN32(1/s) round to fp32 values that encode to
                  different E4M3 codes (quotients within a few fp32 ulps of an
                  E4M3 midpoint);
* ``double_rnd``  the exact quotient, rounded straight to E4M3, differs from the
                  quotient first rounded to fp32 (the fp32 step lands on a tie).

The UE8M0 round-up of the scale is insensitive to the first of these
variants: RN32(1/448) lies above 1/448, and near amax = 448 * 2^p the two
quotients are never on opposite sides of a power of two (checked for every
amax within 6 ulps of 448), so no UE8M0 case separates them.

Every value is written as fp32 bits in hex, so the file is exact.
"""
from __future__ import annotations

import os
import struct
from fractions import Fraction

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "quant_division_cases.txt")


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def bits_f32(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b))[0]


def rn32(x: Fraction) -> Fraction:
    """Round a rational to the nearest fp32 value, ties to even (normal and
    subnormal range; no overflow in these cases)."""
    if x == 0:
        return Fraction(0)
    neg = x < 0
    a = -x if neg else x
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    q = a / quantum
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * quantum
    return -v if neg else v


def as_float(fr: Fraction) -> float:
    v = float(fr)
    assert Fraction(v) == fr
    return v


# E4M3 (OCP, bias 7, max 448): the non-negative finite values in code order,
# from the bit-field definition.
E4M3_POS = []
for code in range(0x7F):
    e, m = code >> 3, code & 7
    E4M3_POS.append(Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
assert all(E4M3_POS[i] < E4M3_POS[i + 1] for i in range(0x7E)) and E4M3_POS[-1] == 448


def enc_e4m3(t: Fraction) -> int:
    """Code of a value already clamped to [-448, 448]; ties to the even code.
    Signed zero is not produced here (the cases have no zero quotients)."""
    neg = t < 0
    a = -t if neg else t
    best = 0
    for c in range(0x7F):
        d, db = abs(E4M3_POS[c] - a), abs(E4M3_POS[best] - a)
        if d < db or (d == db and c % 2 == 0):
            best = c
    return best | (0x80 if neg else 0)


def clamp448(t: Fraction) -> Fraction:
    return max(min(t, Fraction(448)), Fraction(-448))


FLOOR = Fraction(bits_f32(f32_bits(1e-4)))   # fp32(1e-4)


def scale_of(amax: Fraction, ue8m0: bool) -> Fraction:
    s = rn32(max(amax, FLOOR) / 448)
    if ue8m0:
        p = Fraction(1)
        while p < s:
            p *= 2
        while p / 2 >= s:
            p /= 2
        s = p
    return s


def code_of(x: Fraction, s: Fraction) -> int:
    return enc_e4m3(clamp448(rn32(x / s)))


def lcg(seed):
    """Small deterministic generator (64-bit LCG, Knuth's MMIX constants)."""
    state = seed
    while True:
        state = (6364136223846793005 * state + 1442695040888963407) % (1 << 64)
        yield state >> 33


def main():
    rnd = lcg(20240611)
    lines = []

    # ---- scale_div: fp32 amax where amax/448 and amax*RN32(1/448) round apart
    inv448 = rn32(Fraction(1, 448))
    found = 0
    while found < 6:
        amax_bits = 0x3C000000 + next(rnd) % 0x08000000          # amax in [2^-7, 2^9)
        amax = Fraction(bits_f32(amax_bits))
        right = rn32(amax / 448)
        wrong = rn32(amax * inv448)
        if right != wrong:
            s = scale_of(amax, False)
            lines.append(("scale_div_%d" % found, 0, [amax], s, [code_of(amax, s)]))
            found += 1

    # ---- quot_div and double_rnd: x near (E4M3 midpoint) * s for non-dyadic s
    mids = [(E4M3_POS[i] + E4M3_POS[i + 1]) / 2 for i in range(0x7E)]
    quot, dbl = [], []
    tries = 0
    while (len(quot) < 10 or len(dbl) < 4) and tries < 200000:
        tries += 1
        amax = Fraction(bits_f32(0x3E000000 + next(rnd) % 0x06000000))   # amax in [2^-3, 2^9)
        s = scale_of(amax, False)
        inv_s = rn32(1 / s)
        mu = mids[next(rnd) % len(mids)]
        x0 = rn32(mu * s)
        if x0 == 0:
            continue
        for du in range(-3, 4):
            xb = f32_bits(as_float(x0)) + du
            x = Fraction(bits_f32(xb))
            if x <= 0 or x > amax:
                continue
            sign = -1 if next(rnd) % 2 else 1
            xs = sign * x
            right = code_of(xs, s)
            wrong = enc_e4m3(clamp448(rn32(xs * inv_s)))
            direct = enc_e4m3(clamp448(xs / s))
            if right != wrong and len(quot) < 10:
                quot.append((amax, xs, s))
            elif right != direct and len(dbl) < 4:
                dbl.append((amax, xs, s))
    assert len(quot) == 10 and len(dbl) == 4, (len(quot), len(dbl))
    # group three x values per block (the block's amax first)
    for name, cases in (("quot_div", quot), ("double_rnd", dbl)):
        for i, (amax, xs, s) in enumerate(cases):
            lines.append(("%s_%d" % (name, i), 0, [amax, xs], s, [code_of(amax, s), code_of(xs, s)]))

    with open(OUT, "w") as f:
        f.write("# Written by make_quant_division_cases.py (exact rational arithmetic, no oracle call).\n")
        f.write("# 1x128 blocks: the listed values first, the rest of the block zero.  Values and the\n")
        f.write("# scale are fp32 bit patterns; codes are E4M3 bytes, one per listed value.\n")
        f.write("#   name | ue8m0 | values | scale | codes\n")
        for name, ue, xs, s, codes in lines:
            f.write("%-13s| %d | %s | %08X | %s\n" % (
                name, ue, " ".join("%08X" % f32_bits(as_float(v)) for v in xs), f32_bits(as_float(s)),
                " ".join("%02X" % c for c in codes)))
    print(OUT, len(lines), "cases")


if __name__ == "__main__":
    main()
