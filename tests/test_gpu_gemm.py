"""Dense FP8 block-scaled GEMM on the GPU against the CPU oracle.

* Small and ragged shapes (several tiles, M/N tails, K of 1..12 blocks): inputs
  quantized on the host by the oracle, every output element compared.
* The dense LLM-layer shapes at full size, in the launch configuration the
  benchmark times: fp32 draws made on the device, quantized by the library's
  cast kernels; the oracle re-quantizes the sampled A rows and B blocks from the
  same fp32 values (the GPU codes/scales must match them bit for bit) and
  computes the sampled outputs one by one.
* Invariants: determinism, independence of the persistent grid width,
  power-of-two scale linearity, MN-major scale layout.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm
from oracle import quant
from gpu_util import (assert_gemm_close, bits, codes, device, sentinel_like, upload, upload_codes)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_fp8_gemm_amd as dg  # noqa: E402  (fails loudly when the library is missing)


def _host_problem(m, n, k, seed, ue8m0=False):
    w = synth.dense(m, n, k, seed)
    qa, sa = quant.per_token_cast(w.a, ue8m0)
    qb, sb = quant.per_block_cast(w.b, ue8m0)
    return qa, sa, qb, sb


def _gpu_dense(qa, sa, qb, sb, mn_major=False):
    m, n = qa.shape[0], qb.shape[0]
    a, b = upload_codes(qa), upload_codes(qb)
    if mn_major:
        sa_t = upload(np.ascontiguousarray(sa.T)).t()        # strides (1, m)
    else:
        sa_t = upload(sa)
    d = sentinel_like((m, n))
    dg.fp8_gemm_nt((a, sa_t), (b, upload(sb)), d)
    torch.cuda.synchronize()
    return bits(d)


SMALL = [(128, 256, 512), (1, 8, 128), (300, 520, 640), (129, 264, 1536), (64, 2112, 768),
         (520, 392, 256), (256, 1024, 128), (77, 136, 1280)]


@pytest.mark.parametrize("m,n,k", SMALL)
def test_dense_parity_small(m, n, k):
    print(f"dense {m}x{n}x{k}", flush=True)
    qa, sa, qb, sb = _host_problem(m, n, k, seed=m * 7 + n * 3 + k)
    got = _gpu_dense(qa, sa, qb, sb)
    assert_gemm_close(got, ogemm.gemm_nt(qa, sa, qb, sb), f"{m}x{n}x{k}")


def test_config0_workload():
    w = synth.config0()
    qa, sa = quant.per_token_cast(w.a)
    qb, sb = quant.per_block_cast(w.b)
    assert sa.shape == (128, 4) and sb.shape == (2, 4)
    got = _gpu_dense(qa, sa, qb, sb)
    assert_gemm_close(got, ogemm.gemm_nt(qa, sa, qb, sb), "config 0")


def test_mn_major_scales_give_identical_bits():
    qa, sa, qb, sb = _host_problem(300, 264, 512, seed=5)
    assert np.array_equal(_gpu_dense(qa, sa, qb, sb), _gpu_dense(qa, sa, qb, sb, mn_major=True))


def test_ue8m0_scales():
    qa, sa, qb, sb = _host_problem(200, 392, 1024, seed=6, ue8m0=True)
    got = _gpu_dense(qa, sa, qb, sb)
    assert_gemm_close(got, ogemm.gemm_nt(qa, sa, qb, sb), "ue8m0")


def test_power_of_two_scale_linearity_bit_exact():
    qa, sa, qb, sb = _host_problem(160, 264, 512, seed=7)
    base = _gpu_dense(qa, sa, qb, sb)
    up = _gpu_dense(qa, sa * np.float32(8.0), qb, sb)
    down = _gpu_dense(qa, sa, qb, sb * np.float32(0.25))
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)  # noqa: E731
    assert np.array_equal(f(up), f(base) * np.float32(8.0))
    assert np.array_equal(f(down), f(base) * np.float32(0.25))


@pytest.mark.parametrize("m,n,k", [(300, 520, 640), (64, 520, 4096), (1, 8, 128), (256, 512, 1024)])
def test_accumulate_parity(m, n, k):
    # D = RNE_bf16(C + A.B^T); (64, 520, 4096) takes the split-K path, where the
    # last unit to arrive adds C.
    qa, sa, qb, sb = _host_problem(m, n, k, seed=m + 2 * n + k)
    rng = np.random.default_rng(m + n)
    c = (rng.standard_normal((m, n)) * 4).astype(np.float32)
    a, b = (upload_codes(qa), upload(sa)), (upload_codes(qb), upload(sb))
    d = sentinel_like((m, n))
    dg.fp8_gemm_nt(a, b, d, c=upload(c))
    torch.cuda.synchronize()
    assert_gemm_close(bits(d), ogemm.gemm_nt(qa, sa, qb, sb, c), f"acc {m}x{n}x{k}")
    # a zero addend gives the plain result bit for bit; a strided addend (ldc > n) works
    plain = _gpu_dense(qa, sa, qb, sb)
    d0 = sentinel_like((m, n))
    dg.fp8_gemm_nt(a, b, d0, c=torch.zeros((m, n), dtype=torch.float32, device=device()))
    wide = torch.zeros((m, n + 12), dtype=torch.float32, device=device())
    wide[:, :n] = upload(c)
    d1 = sentinel_like((m, n))
    dg.fp8_gemm_nt(a, b, d1, c=wide[:, :n])
    torch.cuda.synchronize()
    assert np.array_equal(bits(d0), plain)
    assert np.array_equal(bits(d1), bits(d))


@pytest.mark.parametrize("m,n,k", [(700, 1032, 768), (96, 1032, 3072)])
def test_deterministic_and_independent_of_grid_width(m, n, k):
    qa, sa, qb, sb = _host_problem(m, n, k, seed=8)
    ref = _gpu_dense(qa, sa, qb, sb)
    assert np.array_equal(ref, _gpu_dense(qa, sa, qb, sb))
    try:
        for cus in (1, 7, 64):
            dg.set_num_cus(cus)
            assert dg.get_num_cus() == cus
            assert np.array_equal(ref, _gpu_dense(qa, sa, qb, sb)), cus
    finally:
        dg.set_num_cus(0)
    assert_gemm_close(ref, ogemm.gemm_nt(qa, sa, qb, sb), f"{m}x{n}x{k}")


# Several tiles per workgroup: 256x256 tiles (two LDS stages) with ragged M and
# N edges; 192x256 tiles (48-row wave bands) with ragged edges and with a last M
# tile whose waves are mostly idle; 128x256 tiles (three stages) with three and
# with two K blocks (fewer blocks than stages).  A narrow grid makes one or five
# workgroups walk all tiles in turn; the result must not change.
CHAINED = [(3800, 4088, 640, 256), (2600, 3104, 640, 192), (4100, 2056, 256, 192), (3000, 2504, 384, 128),
           (2048, 4096, 256, 128)]


@pytest.mark.parametrize("m,n,k,bm", CHAINED)
def test_chained_tiles_on_a_narrow_grid(m, n, k, bm):
    assert dg.tile_config(m, n, k)[0] == bm, "shape no longer picks this tile"
    print(f"chained tiles {m}x{n}x{k}", flush=True)
    qa, sa, qb, sb = _host_problem(m, n, k, seed=m + k)
    ref = _gpu_dense(qa, sa, qb, sb)
    assert_gemm_close(ref, ogemm.gemm_nt(qa, sa, qb, sb), f"{m}x{n}x{k}")
    try:
        for cus in (1, 5):
            dg.set_num_cus(cus)
            assert np.array_equal(ref, _gpu_dense(qa, sa, qb, sb)), cus
    finally:
        dg.set_num_cus(0)


def test_chained_tiles_accumulate_on_a_narrow_grid():
    m, n, k = 2600, 3104, 640
    qa, sa, qb, sb = _host_problem(m, n, k, seed=5)
    c = np.random.default_rng(5).standard_normal((m, n)).astype(np.float32)
    a = (upload_codes(qa), upload(sa))
    b = (upload_codes(qb), upload(sb))

    def run():
        d = sentinel_like((m, n))
        dg.fp8_gemm_nt(a, b, d, c=upload(c))
        torch.cuda.synchronize()
        return bits(d)

    ref = run()
    assert_gemm_close(ref, ogemm.gemm_nt(qa, sa, qb, sb, c), "acc chained")
    try:
        dg.set_num_cus(3)
        assert np.array_equal(ref, run())
    finally:
        dg.set_num_cus(0)


# Small M with deep K: the output has too few tiles for the device, so the K
# blocks are split over several workgroups per output tile (partials summed in
# split order by the last one to arrive).
SPLIT = [(1, 8, 4096), (16, 1536, 2048), (64, 520, 4096), (77, 136, 1280), (128, 2112, 1536),
         (129, 264, 1536), (8, 256, 8192), (200, 1032, 4096)]


@pytest.mark.parametrize("m,n,k", SPLIT)
def test_split_k_parity_and_agreement(m, n, k):
    print(f"split-K {m}x{n}x{k}", flush=True)
    qa, sa, qb, sb = _host_problem(m, n, k, seed=m * 11 + n * 5 + k)
    want = ogemm.gemm_nt(qa, sa, qb, sb)
    need = dg.workspace_size(m, n, k)
    assert need > 0, "shape expected to split"
    ws = torch.zeros(need, dtype=torch.uint8, device=device())
    a, b = (upload_codes(qa), upload(sa)), (upload_codes(qb), upload(sb))
    d = sentinel_like((m, n))
    dg.fp8_gemm_nt(a, b, d, workspace=ws)
    torch.cuda.synchronize()
    split = bits(d)
    assert_gemm_close(split, want, f"split {m}x{n}x{k}")
    # the call left the counter block zero; a second call reuses the workspace
    assert int(ws[:256 * 1024].count_nonzero()) == 0
    d2 = sentinel_like((m, n))
    dg.fp8_gemm_nt(a, b, d2, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(split, bits(d2))
    # no workspace (and a too-small one): the unsplit kernel
    for w in (None, torch.zeros(need - 16, dtype=torch.uint8, device=device())):
        d3 = sentinel_like((m, n))
        dg.fp8_gemm_nt(a, b, d3, workspace=w)
        torch.cuda.synchronize()
        assert_gemm_close(bits(d3), want, f"unsplit {m}x{n}x{k}")


def test_split_k_consecutive_problems_share_the_workspace():
    """Back-to-back calls of different shapes on one stream and one workspace, no host sync between."""
    shapes = [(64, 1032, 2048), (120, 264, 4096), (8, 2048, 1024)]
    probs = [_host_problem(m, n, k, seed=40 + i) for i, (m, n, k) in enumerate(shapes)]
    ws = torch.zeros(max(dg.workspace_size(*s) for s in shapes), dtype=torch.uint8, device=device())
    outs = []
    for qa, sa, qb, sb in probs:
        m, n = qa.shape[0], qb.shape[0]
        d = sentinel_like((m, n))
        dg.fp8_gemm_nt((upload_codes(qa), upload(sa)), (upload_codes(qb), upload(sb)), d, workspace=ws)
        outs.append(d)
    torch.cuda.synchronize()
    for (qa, sa, qb, sb), d in zip(probs, outs):
        assert_gemm_close(bits(d), ogemm.gemm_nt(qa, sa, qb, sb), f"{qa.shape[0]}x{qb.shape[0]}")


# ------------------------------------------------------------------ full size, sampled

def sample_rows(rng, m, count):
    rows = set(rng.choice(m, size=min(m, count), replace=False).tolist()) | {0, m - 1}
    return np.array(sorted(rows))


def sample_blocks_and_cols(rng, n, blocks, per_block):
    nbs = (n + 127) // 128
    chosen = sorted(set(rng.choice(nbs, size=min(nbs, blocks), replace=False).tolist()) | {0, nbs - 1})
    cols = []
    for nb in chosen:
        lo, hi = nb * 128, min(n, nb * 128 + 128)
        cs = set(rng.choice(np.arange(lo, hi), size=min(hi - lo, per_block), replace=False).tolist()) | {lo, hi - 1}
        cols.extend(sorted(cs))
    return chosen, np.array(cols)


def check_sampled(a32, qa, sa, b32, qb, sb, d, rows, blocks, cols, what, ue8m0=False):
    """Oracle re-quantization of the sampled pieces (bit-exact vs the GPU casts)
    and the sampled GEMM outputs (tolerance)."""
    n = b32.shape[0]
    a_rows32 = a32[torch.as_tensor(rows, device=a32.device)].cpu().numpy()
    oqa, osa = quant.per_token_cast(a_rows32, ue8m0)
    gq = codes(qa[torch.as_tensor(rows, device=qa.device)])
    gs = sa[torch.as_tensor(rows, device=sa.device)].cpu().numpy()
    assert np.array_equal(gq, oqa), f"{what}: A codes differ from the oracle quantizer"
    assert np.array_equal(gs.view(np.uint32), osa.view(np.uint32)), f"{what}: A scales differ"
    qb_cols, sb_cols = [], []
    for nb in blocks:
        lo, hi = nb * 128, min(n, nb * 128 + 128)
        blk32 = b32[lo:hi].cpu().numpy()
        oqb, osb = quant.per_block_cast(blk32, ue8m0)
        assert np.array_equal(codes(qb[lo:hi]), oqb), f"{what}: B codes of block {nb} differ"
        assert np.array_equal(sb[nb].cpu().numpy().view(np.uint32), osb[0].view(np.uint32)), f"{what}: B scales"
        sel = cols[(cols >= lo) & (cols < hi)]
        qb_cols.append(oqb[sel - lo])
        sb_cols.append(np.repeat(osb, sel.size, axis=0))
    want = ogemm.gemm_nt_columns(oqa, osa, np.concatenate(qb_cols), np.concatenate(sb_cols))
    ri = torch.as_tensor(rows, device=d.device)
    ci = torch.as_tensor(cols, device=d.device)
    got = bits(d[ri][:, ci])
    return assert_gemm_close(got, want, what)


@pytest.mark.parametrize("idx", range(15))
def test_dense_full_size_sampled(idx):
    m, n, k = synth.config1_shapes()[idx]
    seed = synth.seed_for(1, idx)
    print(f"dense full size {m}x{n}x{k}", flush=True)
    dev = device()
    a32 = synth.draw_activation_device(m, k, seed, dev)
    b32 = synth.draw_weight_device(n, k, seed, 0, dev)
    qa, sa = dg.per_token_cast_fp8(a32)
    qb, sb = dg.per_block_cast_fp8(b32)
    d = sentinel_like((m, n))
    dg.fp8_gemm_nt((qa, sa), (qb, sb), d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    rows = sample_rows(rng, m, 24)
    blocks, cols = sample_blocks_and_cols(rng, n, 3, 12)
    check_sampled(a32, qa, sa, b32, qb, sb, d, rows, blocks, cols, f"{m}x{n}x{k}")
    # every output element was written (no sentinel left, nothing non-finite)
    assert bool(torch.isfinite(d.float()).all())
