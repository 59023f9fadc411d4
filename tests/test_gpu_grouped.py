"""M-grouped contiguous and masked FP8 GEMMs on the GPU against the CPU oracle.

Routing and masking are checked bit for bit (rows the layout excludes keep the
pre-filled sentinel); values are checked to the GEMM tolerance.  Small problems
compare every element with host-quantized inputs; the MoE workloads run at full
size with device-side draws and sampled oracle outputs.  The masked variant is
also captured in a HIP graph and replayed with new masked_m contents.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm
from oracle import quant
from gpu_util import (SENTINEL, assert_gemm_close, bits, codes, device, sentinel_like, upload, upload_codes)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_fp8_gemm_amd as dg  # noqa: E402

from test_gpu_gemm import check_sampled, sample_blocks_and_cols, sample_rows  # noqa: E402


def _quant_groups(b32, ue8m0=False):
    qs, ss = zip(*[quant.per_block_cast(b32[g], ue8m0) for g in range(b32.shape[0])])
    return np.stack(qs), np.stack(ss)


# ------------------------------------------------------------------ contiguous

def _contig_host(num_groups, tokens, n, k, seed, ue8m0=False):
    w = synth.contiguous(num_groups, tokens, [1.0 / num_groups] * num_groups, n, k, seed)
    qa, sa = quant.per_token_cast(w.a, ue8m0)
    qb, sb = _quant_groups(w.b, ue8m0)
    return w, qa, sa, qb, sb


def _gpu_contig(qa, sa, qb, sb, m_indices):
    d = sentinel_like((qa.shape[0], qb.shape[1]))
    dg.m_grouped_fp8_gemm_nt_contiguous((upload_codes(qa), upload(sa)), (upload_codes(qb), upload(sb)), d,
                                        upload(m_indices))
    torch.cuda.synchronize()
    return bits(d)


@pytest.mark.parametrize("groups,tokens,n,k", [(4, 300, 264, 384), (3, 700, 1024, 512), (1, 128, 136, 256)])
def test_contiguous_parity_small(groups, tokens, n, k):
    w, qa, sa, qb, sb = _contig_host(groups, tokens, n, k, seed=tokens + n)
    got = _gpu_contig(qa, sa, qb, sb, w.m_indices)
    pad = w.m_indices < 0
    assert np.all(got[pad] == SENTINEL), "padding rows were written"
    want = ogemm.m_grouped_contiguous(qa, sa, qb, sb, w.m_indices)
    assert_gemm_close(got[~pad], want[~pad], f"contiguous G={groups}")


def test_contiguous_equals_dense_on_each_group_and_groups_are_independent():
    w, qa, sa, qb, sb = _contig_host(3, 500, 392, 512, seed=11)
    got = _gpu_contig(qa, sa, qb, sb, w.m_indices)
    for g in range(3):
        rows = np.nonzero(w.m_indices == g)[0]
        d = sentinel_like((rows.size, qb.shape[1]))
        dg.fp8_gemm_nt((upload_codes(qa[rows]), upload(sa[rows])), (upload_codes(qb[g]), upload(sb[g])), d)
        torch.cuda.synchronize()
        assert np.array_equal(bits(d), got[rows]), g
    qb2 = qb.copy()
    qb2[1] ^= 0x80
    got2 = _gpu_contig(qa, sa, qb2, sb, w.m_indices)
    same = w.m_indices != 1
    assert np.array_equal(got2[same], got[same])


@pytest.mark.parametrize("ue8m0", [False, True])
def test_contiguous_ragged_last_round_split(ue8m0):
    # 12 M tiles x 4 N tiles of 128x256 = 48 tiles.  On a 20-CU grid the two
    # whole rounds (10 M tiles) run in one launch and the last 2 M tiles in a
    # second launch of 128x128 tiles; on 7 CUs it stays one launch.  Every grid
    # must give the bits of the full-width grid, and those match the oracle.
    w, qa, sa, qb, sb = _contig_host(4, 1100, 1024, 512, seed=5, ue8m0=ue8m0)
    assert w.m_indices.size == 1536
    a = (upload_codes(qa), upload(sa))
    b = (upload_codes(qb), upload(sb))
    if ue8m0:
        a = (a[0], dg.pack_ue8m0(a[1]))
        b = (b[0], dg.pack_ue8m0(b[1]))
    mi = upload(w.m_indices)
    pad = w.m_indices < 0
    results = {}
    for cus in (0, 20, 7):
        dg.set_num_cus(cus)
        try:
            d = sentinel_like((qa.shape[0], qb.shape[1]))
            dg.m_grouped_fp8_gemm_nt_contiguous(a, b, d, mi)
            torch.cuda.synchronize()
        finally:
            dg.set_num_cus(0)
        results[cus] = bits(d)
        assert np.all(results[cus][pad] == SENTINEL), f"{cus} CUs: padding rows were written"
    assert np.array_equal(results[20], results[0]) and np.array_equal(results[7], results[0])
    want = ogemm.m_grouped_contiguous(qa, sa, qb, sb, w.m_indices)
    assert_gemm_close(results[0][~pad], want[~pad], "contiguous, split launch")


def test_contiguous_two_launch_plan_graph_replays_with_new_routing():
    # The contiguous call on a 20-CU grid is two launches (see the ragged-round
    # test above).  Captured once, the graph is replayed with the groups of the
    # 128-row segments relabelled each time; every replay must match an eager
    # call on the same grid bit for bit, and the oracle.
    w, qa, sa, qb, sb = _contig_host(4, 1100, 1024, 512, seed=5)
    a = (upload_codes(qa), upload(sa))
    b = (upload_codes(qb), upload(sb))
    mi = upload(w.m_indices)
    d = sentinel_like((qa.shape[0], qb.shape[1]))
    dg.set_num_cus(20)
    try:
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            dg.m_grouped_fp8_gemm_nt_contiguous(a, b, d, mi)      # warm-up outside capture
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            dg.m_grouped_fp8_gemm_nt_contiguous(a, b, d, mi)
        rng = np.random.default_rng(9)
        for rep in range(3):
            perm = rng.permutation(4).astype(np.int32)
            new_idx = np.where(w.m_indices >= 0, perm[np.maximum(w.m_indices, 0)], -1).astype(np.int32)
            mi.copy_(torch.from_numpy(new_idx))
            d.view(torch.int16).fill_(SENTINEL)                    # eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = bits(d)
            eager = _gpu_contig(qa, sa, qb, sb, new_idx)
            assert np.array_equal(got, eager), rep
            pad = new_idx < 0
            assert np.all(got[pad] == SENTINEL)
            want = ogemm.m_grouped_contiguous(qa, sa, qb, sb, new_idx)
            assert_gemm_close(got[~pad], want[~pad], f"replay {rep}")
    finally:
        dg.set_num_cus(0)


def test_contiguous_padding_block_skipped_and_hand_layout():
    # hand-made layout: a fully padded block, a 1-row group, a full block, ragged groups
    k, n, g = 256, 200, 4
    m_indices = np.array([-1] * 128 + [2] + [-1] * 127 + [0] * 128 + [3] * 60 + [-1] * 68, np.int32)
    rng = np.random.default_rng(3)
    a32 = (rng.standard_normal((m_indices.size, k)) * 3).astype(np.float32)
    b32 = rng.standard_normal((g, n, k)).astype(np.float32)
    qa, sa = quant.per_token_cast(a32)
    qb, sb = _quant_groups(b32)
    got = _gpu_contig(qa, sa, qb, sb, m_indices)
    pad = m_indices < 0
    assert np.all(got[pad] == SENTINEL)
    want = ogemm.m_grouped_contiguous(qa, sa, qb, sb, m_indices)
    assert_gemm_close(got[~pad], want[~pad], "hand layout")


def _contig_full(counts, m_indices, n, k, seed, ue8m0, what, rows_per_group_sample):
    dev = device()
    g = counts.size
    m_total = m_indices.size
    valid = torch.as_tensor(np.nonzero(m_indices >= 0)[0], device=dev)
    a32 = torch.zeros((m_total, k), dtype=torch.float32, device=dev)
    a32[valid] = synth.draw_activation_device(int(valid.numel()), k, seed, dev)
    qa, sa = dg.per_token_cast_fp8(a32, ue8m0=ue8m0)
    qb = torch.empty((g, n, k), dtype=torch.float8_e4m3fn, device=dev)
    sb = torch.empty((g, (n + 127) // 128, k // 128), dtype=torch.float32, device=dev)
    for gg in range(g):
        w32 = synth.draw_weight_device(n, k, seed, gg, dev)
        dg.per_block_cast_fp8(w32, ue8m0=ue8m0, q=qb[gg], sf=sb[gg])
        del w32
    d = sentinel_like((m_total, n))
    mi = upload(m_indices)
    dg.m_grouped_fp8_gemm_nt_contiguous((qa, sa), (qb, sb), d, mi)
    torch.cuda.synchronize()
    # padding rows untouched, every valid row written
    pad = torch.as_tensor(m_indices < 0, device=dev)
    assert bool((d.view(torch.int16)[pad] == SENTINEL).all()), f"{what}: padding rows written"
    assert bool(torch.isfinite(d[~pad].float()).all()), f"{what}: valid rows not written"
    # sampled outputs: a few rows of several groups (largest, smallest, first, last)
    rng = np.random.default_rng(seed)
    order = np.argsort(counts)
    groups = sorted(set([int(order[-1]), int(order[0]), 0, g - 1] + rng.choice(g, 3).tolist()))
    for gg in groups:
        rows_g = np.nonzero(m_indices == gg)[0]
        if rows_g.size == 0:
            continue
        rows = rows_g[sample_rows(rng, rows_g.size, rows_per_group_sample)]
        blocks, cols = sample_blocks_and_cols(rng, n, 2, 8)
        b32 = synth.draw_weight_device(n, k, seed, gg, dev)
        check_sampled(a32, qa, sa, b32, qb[gg], sb[gg], d, rows, blocks, cols, f"{what} group {gg}", ue8m0)
        del b32


@pytest.mark.parametrize("idx", [0, 1])
def test_contiguous_full_size_config2(idx):
    counts, m_indices = synth.config2_routing(idx)
    n, k = synth.GROUPED_NK[idx]
    print(f"contiguous G=8 {m_indices.size}x{n}x{k}", flush=True)
    _contig_full(counts, m_indices, n, k, synth.seed_for(2, idx), False, f"config2[{idx}]", 6)


def test_contiguous_full_size_config4_pow2_scales():
    counts, m_indices = synth.config4_routing()
    n, k = synth.CONFIG4_NK
    print(f"contiguous G=256 {m_indices.size}x{n}x{k}", flush=True)
    _contig_full(counts, m_indices, n, k, synth.seed_for(4, 0), True, "config4", 4)


# ------------------------------------------------------------------ masked

def _masked_host(groups, max_m, n, k, seed, masked_m):
    w = synth.masked(groups, max_m, n, k, seed, expected_m=max_m // 2)
    qa, sa = quant.per_token_cast(w.a.reshape(groups * max_m, k))
    qa = qa.reshape(groups, max_m, k)
    sa = sa.reshape(groups, max_m, k // 128)
    qb, sb = _quant_groups(w.b)
    return qa, sa, qb, sb, np.asarray(masked_m, np.int32)


def _gpu_masked(qa, sa, qb, sb, masked_m, expected_m=64):
    g, max_m, _ = qa.shape
    d = sentinel_like((g, max_m, qb.shape[1]))
    dg.m_grouped_fp8_gemm_nt_masked((upload_codes(qa), upload(sa)), (upload_codes(qb), upload(sb)), d,
                                    upload(masked_m), expected_m)
    torch.cuda.synchronize()
    return bits(d)


def test_masked_parity_small_with_edge_counts():
    mm = [0, 1, 127, 128, 129, 200, 300]                 # 300 > max_m clamps to 200
    qa, sa, qb, sb, masked_m = _masked_host(7, 200, 264, 384, seed=21, masked_m=mm)
    got = _gpu_masked(qa, sa, qb, sb, masked_m)
    want = ogemm.m_grouped_masked(qa, sa, qb, sb, masked_m)
    for g, c in enumerate(mm):
        c = min(c, 200)
        assert np.all(got[g, c:] == SENTINEL), f"group {g}: rows beyond masked_m written"
        if c:
            assert_gemm_close(got[g, :c], want[g, :c], f"masked group {g}")


@pytest.mark.parametrize("max_m,counts", [(130, [130, 3, 0, 77]), (100, [100, 65, 64, 1])])
def test_masked_expected_m_is_only_a_hint(max_m, counts):
    """The hint picks the tile (64-row decode tiles up to 64, else 256- or
    128-row tiles by max_m); the output bits must not change."""
    qa, sa, qb, sb, masked_m = _masked_host(4, max_m, 136, 256, seed=22, masked_m=counts)
    ref = _gpu_masked(qa, sa, qb, sb, masked_m, expected_m=1)
    for hint in (64, 65, 128, 4096):
        assert np.array_equal(ref, _gpu_masked(qa, sa, qb, sb, masked_m, expected_m=hint)), hint


def test_masked_decode_tiles_parity():
    """Decode-shaped masked problem on the 64-row tiles: groups of 0..150 rows
    (up to three 64-row tiles), N not a multiple of the 256-column tile."""
    mm = [0, 1, 16, 63, 64, 65, 150]
    qa, sa, qb, sb, masked_m = _masked_host(7, 256, 520, 1280, seed=23, masked_m=mm)
    got = _gpu_masked(qa, sa, qb, sb, masked_m, expected_m=16)
    want = ogemm.m_grouped_masked(qa, sa, qb, sb, masked_m)
    for g, c in enumerate(mm):
        assert np.all(got[g, c:] == SENTINEL), f"group {g}: rows beyond masked_m written"
        if c:
            assert_gemm_close(got[g, :c], want[g, :c], f"decode group {g}")
    assert np.array_equal(got, _gpu_masked(qa, sa, qb, sb, masked_m, expected_m=256))


@pytest.mark.parametrize("idx", [0, 1])
def test_masked_full_size_config3(idx):
    masked_m = synth.config3_masked_m(idx)
    n, k = synth.GROUPED_NK[idx]
    g, max_m = 16, 256
    seed = synth.seed_for(3, idx)
    print(f"masked G=16 max_m=256 {n}x{k}", flush=True)
    dev = device()
    a32 = synth.draw_activation_device(g * max_m, k, seed, dev)
    qa, sa = dg.per_token_cast_fp8(a32)
    qb = torch.empty((g, n, k), dtype=torch.float8_e4m3fn, device=dev)
    sb = torch.empty((g, (n + 127) // 128, k // 128), dtype=torch.float32, device=dev)
    for gg in range(g):
        dg.per_block_cast_fp8(synth.draw_weight_device(n, k, seed, gg, dev), q=qb[gg], sf=sb[gg])
    d = sentinel_like((g, max_m, n))
    dg.m_grouped_fp8_gemm_nt_masked((qa.view(g, max_m, k), sa.view(g, max_m, k // 128)), (qb, sb), d,
                                    upload(masked_m), 128)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    for gg in range(g):
        c = int(masked_m[gg])
        dv = d[gg].view(torch.int16)
        assert bool((dv[c:] == SENTINEL).all()), f"group {gg}: rows beyond masked_m written"
        assert bool(torch.isfinite(d[gg, :c].float()).all())
        if c and gg % 4 == 0:
            rows = sample_rows(rng, c, 6)
            blocks, cols = sample_blocks_and_cols(rng, n, 2, 8)
            b32 = synth.draw_weight_device(n, k, seed, gg, dev)
            check_sampled(a32[gg * max_m:(gg + 1) * max_m], qa[gg * max_m:(gg + 1) * max_m],
                          sa[gg * max_m:(gg + 1) * max_m], b32, qb[gg], sb[gg], d[gg], rows, blocks, cols,
                          f"config3[{idx}] group {gg}")


@pytest.mark.parametrize("idx", [0, 1])
def test_masked_decode_full_size(idx):
    # The decode launch that the benchmark times: G=16 groups of up to 256 rows,
    # at most 32 of them valid, and an expected_m hint of 16 (64-row tiles).  The
    # same call with a hint of 128 (256-row tiles) must give the same bits.
    n, k = synth.GROUPED_NK[idx]
    g, max_m = 16, 256
    seed = synth.seed_for(3, idx)
    masked_m = synth.masked_counts(g, 32, seed + 500)
    print(f"masked decode G=16 max_m=256 rows<=32 {n}x{k}", flush=True)
    dev = device()
    a32 = synth.draw_activation_device(g * max_m, k, seed, dev)
    qa, sa = dg.per_token_cast_fp8(a32)
    qb = torch.empty((g, n, k), dtype=torch.float8_e4m3fn, device=dev)
    sb = torch.empty((g, (n + 127) // 128, k // 128), dtype=torch.float32, device=dev)
    for gg in range(g):
        dg.per_block_cast_fp8(synth.draw_weight_device(n, k, seed, gg, dev), q=qb[gg], sf=sb[gg])
    a = (qa.view(g, max_m, k), sa.view(g, max_m, k // 128))
    d = sentinel_like((g, max_m, n))
    d_big = sentinel_like((g, max_m, n))
    mm = upload(masked_m)
    dg.m_grouped_fp8_gemm_nt_masked(a, (qb, sb), d, mm, 16)
    dg.m_grouped_fp8_gemm_nt_masked(a, (qb, sb), d_big, mm, 128)
    torch.cuda.synchronize()
    assert torch.equal(d.view(torch.int16), d_big.view(torch.int16)), "the hint changed the result"
    rng = np.random.default_rng(seed + 1)
    for gg in range(g):
        c = int(masked_m[gg])
        dv = d[gg].view(torch.int16)
        assert bool((dv[c:] == SENTINEL).all()), f"group {gg}: rows beyond masked_m written"
        assert bool(torch.isfinite(d[gg, :c].float()).all())
        if c and gg % 4 == 1:
            rows = sample_rows(rng, c, 6)
            blocks, cols = sample_blocks_and_cols(rng, n, 2, 8)
            b32 = synth.draw_weight_device(n, k, seed, gg, dev)
            check_sampled(a32[gg * max_m:(gg + 1) * max_m], qa[gg * max_m:(gg + 1) * max_m],
                          sa[gg * max_m:(gg + 1) * max_m], b32, qb[gg], sb[gg], d[gg], rows, blocks, cols,
                          f"decode[{idx}] group {gg}")


def test_masked_graph_capture_replays_with_new_counts():
    qa, sa, qb, sb, masked_m = _masked_host(6, 256, 392, 512, seed=23, masked_m=[10, 256, 0, 100, 129, 7])
    a = (upload_codes(qa), upload(sa))
    b = (upload_codes(qb), upload(sb))
    mm = upload(masked_m)
    d = sentinel_like((6, 256, 392))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        dg.m_grouped_fp8_gemm_nt_masked(a, b, d, mm, 128)   # warm-up outside capture
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dg.m_grouped_fp8_gemm_nt_masked(a, b, d, mm, 128)
    rng = np.random.default_rng(5)
    for rep in range(4):
        new_counts = rng.integers(0, 257, size=6).astype(np.int32)
        mm.copy_(torch.from_numpy(new_counts))
        d.view(torch.int16).fill_(SENTINEL)                # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = bits(d)
        eager = _gpu_masked(qa, sa, qb, sb, new_counts, 128)
        assert np.array_equal(got, eager), rep
        want = ogemm.m_grouped_masked(qa, sa, qb, sb, new_counts)
        for g, c in enumerate(new_counts):
            assert np.all(got[g, c:] == SENTINEL)
            if c:
                assert_gemm_close(got[g, :c], want[g, :c], f"replay {rep} group {g}")
