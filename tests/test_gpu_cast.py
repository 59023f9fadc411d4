"""FP8 casts on the GPU against the oracle quantizer, bit for bit (codes and scale bits).

Covers bf16 and fp32 per-token (1x128) casts with fp32 and power-of-two scales,
the 128x128 weight cast with a partial last block, planted edge rows (all zero,
signed zeros, tiny values, exact ties after division, +-448), the exact-rational
division cases of tests/golden/quant_division_cases.txt, every fp32 value of
magnitude <= 448 through the E4M3 conversion, and every row of the full bf16
[32768, 7168] activation of the Zipf MoE workload.
"""
import concurrent.futures
import os

import numpy as np
import pytest
import torch

import synth
from oracle import e4m3, quant
from gpu_util import codes, device

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_fp8_gemm_amd as dg  # noqa: E402


def _plant_edges(x32: np.ndarray) -> np.ndarray:
    x = x32.copy()
    k = x.shape[1]
    x[0] = 0.0                                             # all-zero row: floor on amax
    x[1] = -0.0                                            # signed zeros
    x[2] = np.float32(1e-30) * np.sign(np.arange(k) % 3 - 1).astype(np.float32)  # tiny, amax floor active
    # amax 448 in every block -> s = 1; then values sitting exactly on E4M3 midpoints
    mids = np.array([1.0625, 1.1875, -2.125, 0.0009765625, 3 * 0.0009765625 / 2, 464.0 - 16, 440.0], np.float32)
    x[3] = np.resize(mids, k)
    x[3, ::128] = 448.0
    x[4] = np.float32(448.0) * np.sign(np.arange(k) % 2 - 0.5).astype(np.float32)
    x[5] = np.float32(3.0e38) * (np.arange(k) % 7 == 0)   # huge amax: tiny quotients underflow to 0 codes
    return x


def _check_cast(x_dev, x32_host, ue8m0, what):
    q, s = dg.per_token_cast_fp8(x_dev, ue8m0=ue8m0)
    torch.cuda.synchronize()
    oq, os_ = quant.per_token_cast(x32_host, ue8m0)
    gq, gs = codes(q), s.cpu().numpy()
    bad = np.argwhere(gq != oq)
    assert bad.size == 0, f"{what}: {bad.shape[0]} codes differ, first at {bad[:4].tolist()}"
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), f"{what}: scales differ"


@pytest.mark.parametrize("ue8m0", [False, True])
def test_per_token_bf16_small_with_edges(ue8m0):
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((96, 1024)) * np.exp2(rng.uniform(-12, 12, (96, 1)))).astype(np.float32)
    x = _plant_edges(x)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    _check_cast(xb.to(device()), xb.float().numpy(), ue8m0, f"bf16 ue8m0={ue8m0}")


@pytest.mark.parametrize("ue8m0", [False, True])
def test_per_token_fp32_small_with_edges(ue8m0):
    rng = np.random.default_rng(32)
    x = (rng.standard_normal((70, 640)) * np.exp2(rng.uniform(-20, 20, (70, 1)))).astype(np.float32)
    x = _plant_edges(x)
    _check_cast(torch.from_numpy(x).to(device()), x, ue8m0, f"fp32 ue8m0={ue8m0}")


def test_per_token_strided_scale_layout():
    rng = np.random.default_rng(33)
    x = rng.standard_normal((40, 512)).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16).to(device())
    q = torch.empty((40, 512), dtype=torch.float8_e4m3fn, device=device())
    s_mn = torch.empty((4, 40), dtype=torch.float32, device=device()).t()   # MN-major scales
    dg.per_token_cast_fp8(xb, q=q, sf=s_mn)
    q2, s2 = dg.per_token_cast_fp8(xb)
    torch.cuda.synchronize()
    assert torch.equal(q.view(torch.uint8), q2.view(torch.uint8)) and torch.equal(s_mn, s2)


@pytest.mark.parametrize("n", [130, 256, 2112])
@pytest.mark.parametrize("ue8m0", [False, True])
def test_per_block_cast(n, ue8m0):
    rng = np.random.default_rng(n)
    w = rng.standard_normal((n, 384)).astype(np.float32)
    w[:128] *= 50.0
    w[-1, :7] = 0.0
    q, s = dg.per_block_cast_fp8(torch.from_numpy(w).to(device()), ue8m0=ue8m0)
    torch.cuda.synchronize()
    oq, os_ = quant.per_block_cast(w, ue8m0)
    assert np.array_equal(codes(q), oq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))


def _boundary_blocks(rng, rows, k):
    """Blocks whose quotients x/s land on and next to E4M3 rounding boundaries
    for many different scales: each row gets its own amax (so its own s); the
    other elements are s * (a midpoint between E4M3 neighbours, or a code value)
    nudged by -2..+2 fp32 ulps, rounded to fp32."""
    from oracle import e4m3 as oe4m3
    vals = np.array(sorted(set(abs(float(v)) for v in oe4m3.DECODE_TABLE if np.isfinite(v))), np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    targets = np.concatenate([mids, vals[1:]])
    x = np.empty((rows, k), np.float32)
    for r in range(rows):
        amax = np.float32(np.exp2(rng.uniform(-20, 20)) * rng.uniform(1, 2))
        s = np.float32(max(amax, np.float32(1e-4)) / np.float32(448.0))
        t = rng.choice(targets, k)
        base = (t * np.float64(s)).astype(np.float32)
        nudge = rng.integers(-2, 3, k).astype(np.int32)
        xi = (base.view(np.int32) + nudge).view(np.float32)
        xi[rng.random(k) < 0.5] *= -1
        xi[::128] = amax                       # the block amax (quotient 448)
        x[r] = np.clip(xi, -amax, amax)
    return x


@pytest.mark.parametrize("ue8m0", [False, True])
def test_per_token_rounding_boundaries_many_scales(ue8m0):
    rng = np.random.default_rng(77)
    x = _boundary_blocks(rng, 256, 2048)
    _check_cast(torch.from_numpy(x).to(device()), x, ue8m0, f"fp32 boundaries ue8m0={ue8m0}")


@pytest.mark.parametrize("ue8m0", [False, True])
def test_per_block_rounding_boundaries(ue8m0):
    rng = np.random.default_rng(78)
    w = _boundary_blocks(rng, 256, 1024)
    q, s = dg.per_block_cast_fp8(torch.from_numpy(w).to(device()), ue8m0=ue8m0)
    torch.cuda.synchronize()
    oq, os_ = quant.per_block_cast(w, ue8m0)
    assert np.array_equal(codes(q), oq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))


def _oracle_cast_rows(x32_chunks, ue8m0):
    """The oracle quantizer over row chunks, several chunks at a time (numpy
    releases the interpreter lock inside its array operations)."""
    workers = min(16, len(os.sched_getaffinity(0)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(lambda c: quant.per_token_cast(c, ue8m0), x32_chunks))


@pytest.mark.parametrize("ue8m0", [False, True])
def test_per_token_full_size_activation_every_row(ue8m0):
    x = synth.config4_cast_input()                         # bf16 [32768, 7168]
    x[:6] = torch.from_numpy(_plant_edges(np.zeros((6, x.shape[1]), np.float32))).to(torch.bfloat16)
    xd = x.to(device())
    q, s = dg.per_token_cast_fp8(xd, ue8m0=ue8m0)
    torch.cuda.synchronize()
    gq, gs = codes(q), s.cpu().numpy()
    step = 1024
    chunks = [x[r:r + step].float().numpy() for r in range(0, x.shape[0], step)]
    for i, (oq, os_) in enumerate(_oracle_cast_rows(chunks, ue8m0)):
        r = i * step
        assert np.array_equal(gq[r:r + step], oq), f"codes differ in rows {r}..{r + step - 1}"
        assert np.array_equal(gs[r:r + step].view(np.uint32), os_.view(np.uint32)), f"scales, rows {r}.."
    print(f"all {x.shape[0]} rows bit-exact (ue8m0={ue8m0})", flush=True)


def _division_cases():
    path = os.path.join(os.path.dirname(__file__), "golden", "quant_division_cases.txt")
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            name, ue, xs, scale, cs = [f.strip() for f in line.split("|")]
            yield (name, bool(int(ue)), np.array([int(v, 16) for v in xs.split()], np.uint32).view(np.float32),
                   int(scale, 16), [int(c, 16) for c in cs.split()])


def test_division_cases_on_the_gpu_casts():
    """Quotients within a few fp32 ulps of E4M3 midpoints and scales where
    amax/448 and amax*RN(1/448) round apart: the GPU's divisions must be the
    correctly rounded ones (expected values derived in exact rational arithmetic)."""
    cases = list(_division_cases())
    x = np.zeros((len(cases), 256), np.float32)
    for i, (_, _, vals, _, _) in enumerate(cases):
        x[i, :vals.size] = vals
        x[i, 128:128 + vals.size] = -vals                # the same block negated
    assert not any(ue for _, ue, _, _, _ in cases)
    q, s = dg.per_token_cast_fp8(torch.from_numpy(x).to(device()))
    w = np.zeros((128 * len(cases), 128), np.float32)
    w[::128] = x[:, :128]
    qw, sw = dg.per_block_cast_fp8(torch.from_numpy(w).to(device()))
    torch.cuda.synchronize()
    gq, gs, gqw, gsw = codes(q), s.cpu().numpy().view(np.uint32), codes(qw), sw.cpu().numpy().view(np.uint32)
    for i, (name, _, vals, scale_bits, want) in enumerate(cases):
        nv = vals.size
        assert gs[i, 0] == scale_bits and gs[i, 1] == scale_bits, name
        assert gq[i, :nv].tolist() == want, name
        assert gq[i, 128:128 + nv].tolist() == [c ^ 0x80 for c in want], name
        assert gsw[i, 0] == scale_bits and gqw[128 * i, :nv].tolist() == want, name


def _e4m3_first_bits():
    """For each non-negative code c, the first fp32 bit pattern the oracle
    encoder maps to c (the encoder is monotone in the value; bisection)."""
    top = int(np.float32(448.0).view(np.uint32))
    enc = lambda b: int(e4m3.encode(np.array([b], np.uint32).view(np.float32).astype(np.float64))[0])  # noqa: E731
    first = [0]
    for c in range(1, 0x7F):
        lo, hi = first[-1], top                            # enc(lo) < c <= enc(hi)
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if enc(mid) >= c:
                hi = mid
            else:
                lo = mid
        assert enc(hi) == c and enc(hi - 1) == c - 1
        first.append(hi)
    return np.array(first + [top + 1], np.int64)


def test_e4m3_conversion_exhaustive():
    """Every fp32 value of magnitude <= 448, both signs, through the fp32
    per-token cast with a block amax of 448 (scale 1, quotient = the value), so
    the codes are the hardware conversion's.  Along increasing bit patterns the
    codes must never decrease and each code must occur exactly as often as the
    oracle encoder's interval for it is long: together that is equality with
    the oracle on every value."""
    first = _e4m3_first_bits()
    want_counts = np.diff(first)                           # values per code 0x00..0x7E
    total = int(first[-1])                                 # bit patterns 0 .. 0x43E00000
    dev = device()
    per_row = 127                                          # column 0 holds the amax 448
    rows = 1 << 20
    for sign in (0, 1):
        counts = torch.zeros(128, dtype=torch.int64, device=dev)
        prev_last = torch.zeros((), dtype=torch.int64, device=dev)
        for start in range(0, total, rows * per_row):
            n_vals = min(rows * per_row, total - start)
            r = -(-n_vals // per_row)
            pat = torch.arange(start, start + r * per_row, dtype=torch.int64, device=dev)
            pat = torch.clamp(pat, max=total - 1)
            if sign:
                pat = pat - (1 << 31)                      # the int32 whose bits are pattern | 0x80000000
            x = torch.empty((r, 128), dtype=torch.float32, device=dev)
            x[:, 0] = 448.0
            x[:, 1:] = pat.to(torch.int32).view(torch.float32).view(r, per_row)
            q, s = dg.per_token_cast_fp8(x)
            assert bool((s == 1.0).all())
            cq = q.view(torch.uint8)[:, 1:].reshape(-1)[:n_vals].to(torch.int64)
            assert bool(((cq >> 7) == sign).all()), "sign bit"
            mag = cq & 0x7F
            assert bool((mag[1:] >= mag[:-1]).all()), f"codes decrease inside the chunk at {start}"
            assert bool(mag[0] >= prev_last), f"codes decrease at the chunk start {start}"
            prev_last = mag[-1]
            counts += torch.bincount(mag, minlength=128)
            del x, q, s, pat, cq, mag
        got = counts.cpu().numpy()
        assert got[0x7F] == 0
        bad = np.nonzero(got[:0x7F] != want_counts)[0]
        assert bad.size == 0, f"sign {sign}: code counts differ at {[hex(int(c)) for c in bad[:8]]}"
        print(f"sign {sign}: {total} values, all codes match the oracle", flush=True)
