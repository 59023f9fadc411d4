"""FP8 casts on the GPU against the oracle quantizer, bit for bit (codes and scale bits).

Covers bf16 and fp32 per-token (1x128) casts with fp32 and power-of-two scales,
the 128x128 weight cast with a partial last block, planted edge rows (all zero,
signed zeros, tiny values, exact ties after division, +-448), and the full
bf16 [32768, 7168] activation of the Zipf MoE workload (sampled rows plus the
planted ones).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import quant
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


@pytest.mark.parametrize("ue8m0", [False, True])
def test_per_token_full_size_activation_sampled(ue8m0):
    x = synth.config4_cast_input()                         # bf16 [32768, 7168]
    x[:6] = torch.from_numpy(_plant_edges(np.zeros((6, x.shape[1]), np.float32))).to(torch.bfloat16)
    xd = x.to(device())
    q, s = dg.per_token_cast_fp8(xd, ue8m0=ue8m0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(44)
    rows = np.array(sorted(set(rng.choice(x.shape[0], 2048, replace=False).tolist()) | set(range(6)) | {x.shape[0] - 1}))
    x32 = x[torch.as_tensor(rows)].float().numpy()
    oq, os_ = quant.per_token_cast(x32, ue8m0)
    ri = torch.as_tensor(rows, device=device())
    assert np.array_equal(codes(q[ri]), oq)
    assert np.array_equal(s[ri].cpu().numpy().view(np.uint32), os_.view(np.uint32))
