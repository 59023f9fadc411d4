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

from test_gpu_gemm import assert_exact_rate, check_sampled, sample_blocks_and_cols, sample_rows  # noqa: E402


def _quant_groups(b32, ue8m0=False):
    qs, ss = zip(*[quant.per_block_cast(b32[g], ue8m0) for g in range(b32.shape[0])])
    return np.stack(qs), np.stack(ss)


# ------------------------------------------------------------------ contiguous

def _contig_host(num_groups, tokens, n, k, seed, ue8m0=False):
    w = synth.contiguous(num_groups, tokens, [1.0 / num_groups] * num_groups, n, k, seed)
    qa, sa = quant.per_token_cast(w.a, ue8m0)
    qb, sb = _quant_groups(w.b, ue8m0)
    return w, qa, sa, qb, sb


def _gpu_contig(qa, sa, qb, sb, m_indices, workspace="auto", packed=False):
    d = sentinel_like((qa.shape[0], qb.shape[1]))
    a_s, b_s = upload(sa), upload(sb)
    if packed:
        a_s, b_s = dg.pack_ue8m0(a_s), dg.pack_ue8m0(b_s)
    dg.m_grouped_fp8_gemm_nt_contiguous((upload_codes(qa), a_s), (upload_codes(qb), b_s), d,
                                        upload(m_indices), workspace=workspace)
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
    # without a workspace no K is split, so every row is computed as the dense GEMM computes it
    w, qa, sa, qb, sb = _contig_host(3, 500, 392, 512, seed=11)
    got = _gpu_contig(qa, sa, qb, sb, w.m_indices, workspace=None)
    for g in range(3):
        rows = np.nonzero(w.m_indices == g)[0]
        d = sentinel_like((rows.size, qb.shape[1]))
        dg.fp8_gemm_nt((upload_codes(qa[rows]), upload(sa[rows])), (upload_codes(qb[g]), upload(sb[g])), d)
        torch.cuda.synchronize()
        assert np.array_equal(bits(d), got[rows]), g
    qb2 = qb.copy()
    qb2[1] ^= 0x80
    got2 = _gpu_contig(qa, sa, qb2, sb, w.m_indices, workspace=None)
    same = w.m_indices != 1
    assert np.array_equal(got2[same], got[same])


class _contig_plan:
    """Force a contiguous plan (1 paired, 2 one tile per block) inside a with-block."""

    def __init__(self, plan):
        self.plan = plan

    def __enter__(self):
        dg.set_contiguous_plan(self.plan)

    def __exit__(self, *exc):
        dg.set_contiguous_plan(0)


@pytest.mark.parametrize("ue8m0", [False, True])
def test_contiguous_ragged_last_round_split(ue8m0):
    # The one-tile-per-block plan: 12 M tiles x 4 N tiles of 128x256 = 48
    # tiles.  On a 20-CU grid the two whole rounds (10 M tiles) run in one
    # launch and the last 2 M tiles in a second launch of 128x128 tiles; on 7
    # CUs it stays one launch.  Every grid must give the bits of the full-width
    # grid, and those match the oracle.
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
            with _contig_plan(2):
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


def _segments_layout(segments):
    """m_indices from (group, blocks, valid rows of the last block) segments;
    group -1 gives padding-only blocks."""
    parts = []
    for g, nb, last_valid in segments:
        for b in range(nb):
            valid = 128 if (b < nb - 1 or g < 0) else last_valid
            parts.append(np.full(valid, g, np.int32))
            parts.append(np.full(128 - valid, -1, np.int32))
    return np.concatenate(parts)


def _random_problem(m_total, groups, n, k, seed):
    """Codes of N(0,1) * 32 values (torch's CPU E4M3 conversion, fast for big
    layouts) and random power-of-two-ish scales.  Uniformly random codes would
    span 2^35 in product magnitude, far beyond what quantized data holds."""
    rng = np.random.default_rng(seed)

    def codes(shape):
        x = torch.from_numpy((rng.standard_normal(shape) * 32).astype(np.float32))
        return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    qa = codes((m_total, k))
    sa = np.exp2(rng.uniform(-12, -4, size=(m_total, k // 128))).astype(np.float32)
    qb = codes((groups, n, k))
    sb = np.exp2(rng.uniform(-12, -4, size=(groups, (n + 127) // 128, k // 128))).astype(np.float32)
    return qa, sa, qb, sb


PAIR_LAYOUTS = {
    # odd-aligned starts, segments of 1, 2, 3 blocks, a padding-only block
    # between two blocks of one group, adjacent groups, a trailing single
    "short_segments": [(0, 3, 100), (1, 1, 1), (2, 2, 128), (3, 5, 64), (-1, 1, 0), (3, 1, 7), (0, 2, 128),
                       (1, 4, 90), (2, 1, 128)],
    # long segments crossing the 32-block chunks each lane of the scan walks
    "long_segments": [(g % 4, 17 + 7 * g, 128 - 9 * g) for g in range(8)] + [(-1, 2, 0)],
}


@pytest.mark.parametrize("name", sorted(PAIR_LAYOUTS))
def test_contiguous_pair_plan_layouts(name):
    """Pairs of consecutive blocks of a group run as 256-row tiles, leftover
    blocks as 128-row tiles: padding rows untouched, values within the oracle's
    tolerance, and the same bits as the one-tile-per-block plan and as a narrow
    grid (one workgroup walking every tile)."""
    m_indices = _segments_layout(PAIR_LAYOUTS[name])
    groups = 4
    nb = m_indices.size // 128
    assert nb >= 2 * groups
    n, k = 264, 384
    qa, sa, qb, sb = _random_problem(m_indices.size, groups, n, k, seed=nb)
    with _contig_plan(1):
        got = _gpu_contig(qa, sa, qb, sb, m_indices)
    pad = m_indices < 0
    assert np.all(got[pad] == SENTINEL), "padding rows written"
    want = ogemm.m_grouped_contiguous(qa, sa, qb, sb, m_indices)
    assert_gemm_close(got[~pad], want[~pad], name)
    with _contig_plan(2):
        assert np.array_equal(_gpu_contig(qa, sa, qb, sb, m_indices), got)
    try:
        dg.set_num_cus(1)
        with _contig_plan(1):
            assert np.array_equal(_gpu_contig(qa, sa, qb, sb, m_indices), got)
    finally:
        dg.set_num_cus(0)


def _paired_blocks(m_indices):
    """Blocks the paired plan covers with 256-row tiles: in each run of
    consecutive blocks of one group (a block's group is that of its first row;
    padding blocks end a run), blocks pair up from the start of the run."""
    nb = m_indices.size // 128
    grp = m_indices[::128]
    paired = np.zeros(nb, bool)
    b = 0
    while b < nb:
        if grp[b] < 0:
            b += 1
            continue
        e = b
        while e + 1 < nb and grp[e + 1] == grp[b]:
            e += 1
        length = e - b + 1
        paired[b:b + length // 2 * 2] = True
        b = e + 1
    return paired


SPLIT_LAYOUTS = {
    # 3 pairs and 4 leftover blocks over 4 groups, ragged last blocks, a padding block
    "mixed": [(0, 3, 100), (1, 1, 77), (2, 2, 128), (3, 1, 5), (-1, 1, 0), (1, 3, 128)],
    # one block per group: everything runs in the second launch
    "all_leftover": [(0, 1, 128), (1, 1, 64), (2, 1, 1), (3, 1, 128)],
}


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("name", sorted(SPLIT_LAYOUTS))
def test_contiguous_split_leftover_blocks(name, packed):
    """With a workspace, the paired plan's second launch splits K over the CUs
    its few tiles leave idle (the split is chosen on the device from the
    number of leftover blocks).  Rows of paired blocks keep the bits of the
    unsplit call; every row is within the oracle's tolerance; the result is
    deterministic, independent of the grid width, and (power-of-two scales)
    the same with packed UE8M0 words as with fp32 words."""
    m_indices = _segments_layout(SPLIT_LAYOUTS[name])
    groups, n, k = 4, 520, 2048
    qa, sa, qb, sb = _random_problem(m_indices.size, groups, n, k, seed=m_indices.size)
    if packed:
        sa, sb = np.exp2(np.round(np.log2(sa))).astype(np.float32), np.exp2(np.round(np.log2(sb))).astype(np.float32)
    with _contig_plan(1):
        need = dg.contiguous_workspace_size(m_indices.size, n, k, groups)
        assert need > 0, "no split planned"
        print(f"contiguous split {name} packed={packed}", flush=True)
        split = _gpu_contig(qa, sa, qb, sb, m_indices, packed=packed)
        again = _gpu_contig(qa, sa, qb, sb, m_indices, packed=packed)
        unsplit = _gpu_contig(qa, sa, qb, sb, m_indices, workspace=None, packed=packed)
        # a workspace one byte short of the plan's need: the call runs unsplit
        short = torch.zeros(need - 1, dtype=torch.uint8, device=device())
        assert np.array_equal(_gpu_contig(qa, sa, qb, sb, m_indices, workspace=short, packed=packed), unsplit)
        try:
            dg.set_num_cus(3)
            narrow = _gpu_contig(qa, sa, qb, sb, m_indices, packed=packed)
        finally:
            dg.set_num_cus(0)
        if packed:
            fp32_words = _gpu_contig(qa, sa, qb, sb, m_indices)
            assert np.array_equal(split, fp32_words)
    assert np.array_equal(split, again) and np.array_equal(split, narrow)
    pad = m_indices < 0
    assert np.all(split[pad] == SENTINEL), "padding rows written"
    paired_rows = np.repeat(_paired_blocks(m_indices), 128)
    assert np.array_equal(split[paired_rows], unsplit[paired_rows])
    want = ogemm.m_grouped_contiguous(qa, sa, qb, sb, m_indices)
    assert_gemm_close(split[~pad], want[~pad], f"split {name}")
    assert_gemm_close(unsplit[~pad], want[~pad], f"unsplit {name}")


def test_contiguous_split_plan_graph_replays_with_new_routing():
    """The paired plan with split leftover blocks, captured once as a HIP graph
    and replayed with routings of the same 8 blocks whose leftover-block count
    differs (2, 4, 0, 1), so that the split the kernel picks on the device
    changes between replays.  Every replay must equal an eager call bit for bit
    and match the oracle; the workspace's counters must come back zero."""
    groups, n, k = 4, 520, 2048
    routings = [[(0, 3, 128), (1, 2, 90), (2, 1, 128), (3, 2, 7)],
                [(0, 1, 128), (1, 1, 64), (2, 1, 128), (3, 5, 100)],
                [(3, 2, 128), (2, 2, 128), (1, 2, 1), (0, 2, 128)],
                [(1, 6, 128), (0, 1, 33), (2, 1, 128)]]
    layouts = [_segments_layout(r) for r in routings]
    m_total = layouts[0].size
    assert all(l.size == m_total for l in layouts)
    qa, sa, qb, sb = _random_problem(m_total, groups, n, k, seed=77)
    a = (upload_codes(qa), upload(sa))
    b = (upload_codes(qb), upload(sb))
    mi = upload(layouts[0])
    d = sentinel_like((m_total, n))
    with _contig_plan(1):
        need = dg.contiguous_workspace_size(m_total, n, k, groups)
        assert need > 0
        ws = torch.zeros(need, dtype=torch.uint8, device=device())
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            dg.m_grouped_fp8_gemm_nt_contiguous(a, b, d, mi, workspace=ws)     # warm-up outside capture
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            dg.m_grouped_fp8_gemm_nt_contiguous(a, b, d, mi, workspace=ws)
        for rep, layout in enumerate(layouts[1:] + layouts[:1]):
            print(f"split-plan graph replay {rep}: {int((~_paired_blocks(layout) & (layout[::128] >= 0)).sum())} "
                  "leftover blocks", flush=True)
            mi.copy_(torch.from_numpy(layout))
            d.view(torch.int16).fill_(SENTINEL)                    # eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = bits(d)
            assert int(ws[:256 * 1024].view(torch.int32).abs().sum().item()) == 0, "counters not left zero"
            eager = _gpu_contig(qa, sa, qb, sb, layout, workspace=ws)
            assert np.array_equal(got, eager), rep
            pad = layout < 0
            assert np.all(got[pad] == SENTINEL)
            want = ogemm.m_grouped_contiguous(qa, sa, qb, sb, layout)
            assert_gemm_close(got[~pad], want[~pad], f"split-plan replay {rep}")


@pytest.mark.parametrize("nblocks", [2048, 2049])
def test_contiguous_pair_plan_largest_layout(nblocks):
    """2048 blocks is the largest layout the paired plan takes (its tile list
    lives in LDS); 2049 blocks runs the one-tile-per-block plan.  Segments of
    1..11 blocks over 8 groups, cycling, so that pairs and singles cross every
    32-block chunk of the device-side scan.  Sampled rows of every group."""
    segs, total, i = [], 0, 0
    while total < nblocks:
        length = min(1 + (i * 7) % 11, nblocks - total)
        segs.append((i % 8, length, 128 - (i * 13) % 128))
        total += length
        i += 1
    m_indices = _segments_layout(segs)
    assert m_indices.size == nblocks * 128
    n, k = 64, 128
    qa, sa, qb, sb = _random_problem(m_indices.size, 8, n, k, seed=nblocks)
    with _contig_plan(1):          # taken up to 2048 blocks; beyond, plan 2 regardless
        got = _gpu_contig(qa, sa, qb, sb, m_indices)
    pad = m_indices < 0
    assert np.all(got[pad] == SENTINEL), "padding rows written"
    rows = np.nonzero(~pad)[0][::97]
    want = ogemm.m_grouped_contiguous(qa[rows], sa[rows], qb, sb, m_indices[rows])
    assert_gemm_close(got[rows], want, f"{nblocks} blocks")
    assert bool(np.isfinite((got[~pad].astype(np.uint32) << 16).view(np.float32)).all()), "a valid row was not written"


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


def _contig_full(counts, m_indices, n, k, seed, ue8m0, what, rows_per_group_sample, packed=False):
    """Full-size contiguous run as the benchmark does it: A scales written by the
    cast in the MN-major layout; with ``packed`` both scale arrays are then
    packed to UE8M0 words (A's words MN-major) and the packed GEMM runs."""
    dev = device()
    g = counts.size
    m_total = m_indices.size
    valid = torch.as_tensor(np.nonzero(m_indices >= 0)[0], device=dev)
    a32 = torch.zeros((m_total, k), dtype=torch.float32, device=dev)
    a32[valid] = synth.draw_activation_device(int(valid.numel()), k, seed, dev)
    sa_mn = torch.empty((k // 128, m_total), dtype=torch.float32, device=dev).t()
    qa, sa = dg.per_token_cast_fp8(a32, ue8m0=ue8m0, sf=sa_mn)
    qb = torch.empty((g, n, k), dtype=torch.float8_e4m3fn, device=dev)
    sb = torch.empty((g, (n + 127) // 128, k // 128), dtype=torch.float32, device=dev)
    for gg in range(g):
        w32 = synth.draw_weight_device(n, k, seed, gg, dev)
        dg.per_block_cast_fp8(w32, ue8m0=ue8m0, q=qb[gg], sf=sb[gg])
        del w32
    d = sentinel_like((m_total, n))
    mi = upload(m_indices)
    if packed:
        words = (k // 128 + 3) // 4
        pa = dg.pack_ue8m0(sa, out=torch.empty((words, m_total), dtype=torch.int32, device=dev).t())
        pb = dg.pack_ue8m0(sb)
        dg.m_grouped_fp8_gemm_nt_contiguous((qa, pa), (qb, pb), d, mi)
    else:
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
    stats = []
    for gg in groups:
        rows_g = np.nonzero(m_indices == gg)[0]
        if rows_g.size == 0:
            continue
        rows = rows_g[sample_rows(rng, rows_g.size, rows_per_group_sample)]
        blocks, cols = sample_blocks_and_cols(rng, n, 2, 8)
        b32 = synth.draw_weight_device(n, k, seed, gg, dev)
        stats.append(check_sampled(a32, qa, sa, b32, qb[gg], sb[gg], d, rows, blocks, cols,
                                   f"{what} group {gg}", ue8m0))
        del b32
    # most outputs are the exactly rounded result, as for the dense shapes
    assert_exact_rate(stats, 0.95, what)


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


def test_contiguous_full_size_config4_packed_ue8m0():
    counts, m_indices = synth.config4_routing()
    n, k = synth.CONFIG4_NK
    print(f"contiguous G=256 packed UE8M0 {m_indices.size}x{n}x{k}", flush=True)
    _contig_full(counts, m_indices, n, k, synth.seed_for(4, 0), True, "config4 packed", 4, packed=True)


# ------------------------------------------------------------------ masked

def _random_contiguous_cases(count, seed):
    """Seeded grouped layouts: 1-12 groups, 1-2000 tokens routed with Dirichlet
    expert popularity (empty experts included), N a multiple of 8, K a multiple
    of 128."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        g = int(rng.integers(1, 13))
        probs = rng.dirichlet(np.full(g, 0.6)).tolist()
        cases.append((g, int(rng.integers(1, 2001)), 8 * int(rng.integers(1, 200)), 128 * int(rng.integers(1, 25)),
                      probs, int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("case", _random_contiguous_cases(8, seed=77))
def test_contiguous_random_layouts(case):
    """The cost model's plan (paired 256-row tiles, split-K leftover blocks or
    one tile per block) on random routings: every routed row matches the oracle
    and every padding row keeps the sentinel."""
    groups, tokens, n, k, probs, seed = case
    w = synth.contiguous(groups, tokens, probs, n, k, seed)
    print(f"contiguous random G={groups} tokens={tokens} rows={w.m_indices.size} {n}x{k} "
          f"counts={w.counts.tolist()}", flush=True)
    qa, sa = quant.per_token_cast(w.a)
    qb, sb = _quant_groups(w.b)
    got = _gpu_contig(qa, sa, qb, sb, w.m_indices)
    pad = w.m_indices < 0
    assert np.all(got[pad] == SENTINEL), "padding rows were written"
    if (~pad).any():
        want = ogemm.m_grouped_contiguous(qa, sa, qb, sb, w.m_indices)
        assert_gemm_close(got[~pad], want[~pad], f"contiguous random G={groups}")


def _random_masked_cases(count, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        g = int(rng.integers(1, 25))
        max_m = int(rng.integers(1, 401))
        mm = rng.integers(0, max_m + 1, size=g)
        mm[rng.random(g) < 0.15] = 0
        mm[rng.random(g) < 0.15] = max_m
        cases.append((g, max_m, 8 * int(rng.integers(1, 160)), 128 * int(rng.integers(1, 17)), mm.tolist(),
                      int(rng.choice([1, 16, 64, 65, 128, 4096])), int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("case", _random_masked_cases(8, seed=78))
def test_masked_random_counts(case):
    """Random group counts, row bounds, masked_m and expected_m hints: rows below
    masked_m match the oracle, rows at or past it keep the sentinel."""
    groups, max_m, n, k, mm, hint, seed = case
    print(f"masked random G={groups} max_m={max_m} {n}x{k} hint {hint} masked_m={mm}", flush=True)
    qa, sa, qb, sb, masked_m = _masked_host(groups, max_m, n, k, seed=seed, masked_m=mm)
    got = _gpu_masked(qa, sa, qb, sb, masked_m, expected_m=hint)
    rows = np.asarray(mm)
    valid = np.arange(max_m)[None, :] < rows[:, None]
    assert np.all(got[~valid] == SENTINEL), "rows at or past masked_m were written"
    if valid.any():
        want = ogemm.m_grouped_masked(qa, sa, qb, sb, masked_m)
        assert_gemm_close(got[valid], want[valid], f"masked random G={groups}")


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


def test_grouped_offsets_near_the_32bit_limit():
    """One group's A rows are addressed with 32-bit per-lane byte offsets (rows x
    leading dimension < 2^32); groups are 64-bit apart.  Contiguous: 4096 rows
    1 MiB - 16 bytes apart, the last just under 4 GiB from the first.  Masked:
    two groups of 4095 rows 1 MiB apart, the second group 4 GiB after the first.
    Both match the oracle on every valid row; one M tile (contiguous) or one row
    per group (masked) more is rejected before any launch, leaving D untouched."""
    dev = device()
    n, k = 256, 512
    b32 = np.stack([synth.dense(1, n, k, 90 + g).b for g in range(4)])
    qb, sb = _quant_groups(b32)
    b = (upload_codes(qb), upload(sb))

    # contiguous: segments of 1000, 1500, 0 and 1450 tokens, each padded to 128 rows
    m_indices = np.concatenate([np.r_[np.full(c, g), np.full(-c % 128, -1)] for g, c in
                                enumerate([1000, 1500, 0, 1450])]).astype(np.int32)
    m_total, lda = m_indices.size, (1 << 20) - 16
    assert m_total == 4096 and (m_total - 1) * lda + k < 2 ** 32 <= (m_total + 128) * lda
    print(f"contiguous {m_total}x{n}x{k}, A rows {lda} bytes apart", flush=True)
    a32 = synth.dense(m_total, 8, k, 91).a
    a32[m_indices < 0] = 0.0
    qa, sa = quant.per_token_cast(a32)
    buf = torch.zeros((m_total + 127) * lda + k, dtype=torch.uint8, device=dev)
    a_rows = buf.as_strided((m_total, k), (lda, 1))
    a_rows.copy_(torch.from_numpy(qa).to(dev))
    d = sentinel_like((m_total, n))
    dg.m_grouped_fp8_gemm_nt_contiguous((a_rows.view(torch.float8_e4m3fn), upload(sa)), b, d, upload(m_indices))
    torch.cuda.synchronize()
    got, valid = bits(d), m_indices >= 0
    assert np.all(got[~valid] == SENTINEL), "padding rows were written"
    want = ogemm.m_grouped_contiguous(qa, sa, qb, sb, m_indices)
    assert_gemm_close(got[valid], want[valid], "contiguous at the offset limit")
    more = np.r_[m_indices, np.full(128, 1, np.int32)]
    d = sentinel_like((m_total + 128, n))
    with pytest.raises(dg.DgError) as err:
        dg.m_grouped_fp8_gemm_nt_contiguous((buf.as_strided((m_total + 128, k), (lda, 1)).view(torch.float8_e4m3fn),
                                             upload(np.ones((m_total + 128, k // 128), np.float32))), b, d,
                                            upload(more))
    assert err.value.status == dg.DG_ERROR_NOT_SUPPORTED
    del buf, a_rows

    # masked: group stride 2^32 bytes, rows 2^20 bytes apart
    g, max_m, lda, gs = 2, 4095, 1 << 20, 1 << 32
    assert (max_m - 1) * lda + k < 2 ** 32 <= (max_m + 1) * lda
    print(f"masked {g}x{max_m}x{n}x{k}, A rows {lda} and groups {gs} bytes apart", flush=True)
    masked_m = np.array([4095, 2500], np.int32)
    a32 = synth.dense(g * max_m, 8, k, 92).a.reshape(g, max_m, k)
    qa, sa = quant.per_token_cast(a32.reshape(-1, k))
    qa, sa = qa.reshape(g, max_m, k), sa.reshape(g, max_m, k // 128)
    buf = torch.zeros((g - 1) * gs + max_m * lda + k, dtype=torch.uint8, device=dev)
    a_rows = buf.as_strided((g, max_m, k), (gs, lda, 1))
    a_rows.copy_(torch.from_numpy(qa).to(dev))
    d = sentinel_like((g, max_m, n))
    dg.m_grouped_fp8_gemm_nt_masked((a_rows.view(torch.float8_e4m3fn), upload(sa)), (b[0][:g], b[1][:g]), d,
                                    upload(masked_m), 2048)
    torch.cuda.synchronize()
    got = bits(d)
    want = ogemm.m_grouped_masked(qa, sa, qb[:g], sb[:g], masked_m)
    for gg, c in enumerate(masked_m):
        assert np.all(got[gg, c:] == SENTINEL), f"group {gg}: rows beyond masked_m written"
        assert_gemm_close(got[gg, :c], want[gg, :c], f"masked group {gg} at the offset limit")
    d = sentinel_like((g, max_m + 1, n))
    with pytest.raises(dg.DgError) as err:
        dg.m_grouped_fp8_gemm_nt_masked((buf.as_strided((g, max_m + 1, k), (gs, lda, 1)).view(torch.float8_e4m3fn),
                                         upload(np.ones((g, max_m + 1, k // 128), np.float32))),
                                        (b[0][:g], b[1][:g]), d, upload(masked_m), 2048)
    assert err.value.status == dg.DG_ERROR_NOT_SUPPORTED
    torch.cuda.synchronize()
    assert bool((d.view(torch.int16) == SENTINEL).all()), "a rejected call wrote D"


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


def test_masked_largest_group_count():
    # 1024 groups, the most the device-side prefix over masked_m holds: counts
    # spread over every lane's share of the prefix, with empty groups, full
    # groups, and values the kernel clamps (negative, above max_m); both tile
    # heights give the same bits, and every group matches the oracle.
    groups, max_m, n, k = 1024, 64, 64, 128
    rng = np.random.default_rng(31)
    mm = rng.integers(0, max_m + 1, size=groups)
    mm[rng.random(groups) < 0.1] = 0
    mm[rng.random(groups) < 0.1] = max_m
    mm[5], mm[700], mm[1023] = -3, max_m + 40, 1
    qa, sa, qb, sb, masked_m = _masked_host(groups, max_m, n, k, seed=32, masked_m=mm)
    print(f"masked {groups} groups, {int(np.clip(mm, 0, max_m).sum())} rows", flush=True)
    got = _gpu_masked(qa, sa, qb, sb, masked_m, expected_m=16)
    assert np.array_equal(_gpu_masked(qa, sa, qb, sb, masked_m, expected_m=128), got)
    want = ogemm.m_grouped_masked(qa, sa, qb, sb, masked_m)
    rows = np.clip(mm, 0, max_m)
    valid = np.arange(max_m)[None, :] < rows[:, None]
    assert np.all(got[~valid] == SENTINEL), "rows beyond masked_m written"
    assert_gemm_close(got[valid], want[valid], "1024 masked groups")


@pytest.mark.parametrize("expected_m", [16, 128])
def test_masked_schedule_does_not_change_the_bits(expected_m):
    """Which workgroup runs which masked tile depends on the group layout and on
    the grid width.  Permuting the groups (operands and counts alike), or
    narrowing the grid so that each workgroup walks many tiles, must permute or
    keep the output bits and nothing else.  Counts include ties, empty groups
    and groups of two 256-row tiles."""
    mm = np.array([300, 0, 77, 257, 77, 1, 256, 300, 0, 129, 64, 77], np.int32)
    groups, max_m, n, k = mm.size, 300, 520, 384
    qa, sa, qb, sb, masked_m = _masked_host(groups, max_m, n, k, seed=24, masked_m=mm)
    ref = _gpu_masked(qa, sa, qb, sb, masked_m, expected_m)
    want = ogemm.m_grouped_masked(qa, sa, qb, sb, masked_m)
    for g, c in enumerate(mm):
        assert np.all(ref[g, c:] == SENTINEL), f"group {g}: rows beyond masked_m written"
        if c:
            assert_gemm_close(ref[g, :c], want[g, :c], f"masked group {g}")
    perm = np.random.default_rng(25).permutation(groups)
    got = _gpu_masked(qa[perm], sa[perm], qb[perm], sb[perm], masked_m[perm], expected_m)
    assert np.array_equal(got, ref[perm]), "group order changed the bits"
    for cus in (1, 3, 7, 20):
        try:
            dg.set_num_cus(cus)
            print(f"masked schedule: grid of {cus}", flush=True)
            narrow = _gpu_masked(qa, sa, qb, sb, masked_m, expected_m)
        finally:
            dg.set_num_cus(0)
        assert np.array_equal(narrow, ref), f"grid of {cus} changed the bits"


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
    stats = []
    for gg in range(g):
        c = int(masked_m[gg])
        dv = d[gg].view(torch.int16)
        assert bool((dv[c:] == SENTINEL).all()), f"group {gg}: rows beyond masked_m written"
        assert bool(torch.isfinite(d[gg, :c].float()).all())
        if c and gg % 4 == 0:
            rows = sample_rows(rng, c, 6)
            blocks, cols = sample_blocks_and_cols(rng, n, 2, 8)
            b32 = synth.draw_weight_device(n, k, seed, gg, dev)
            stats.append(check_sampled(a32[gg * max_m:(gg + 1) * max_m], qa[gg * max_m:(gg + 1) * max_m],
                                       sa[gg * max_m:(gg + 1) * max_m], b32, qb[gg], sb[gg], d[gg], rows,
                                       blocks, cols, f"config3[{idx}] group {gg}"))
    assert_exact_rate(stats, 0.95, f"config3[{idx}]")


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
    stats = []
    for gg in range(g):
        c = int(masked_m[gg])
        dv = d[gg].view(torch.int16)
        assert bool((dv[c:] == SENTINEL).all()), f"group {gg}: rows beyond masked_m written"
        assert bool(torch.isfinite(d[gg, :c].float()).all())
        if c and gg % 4 == 1:
            rows = sample_rows(rng, c, 6)
            blocks, cols = sample_blocks_and_cols(rng, n, 2, 8)
            b32 = synth.draw_weight_device(n, k, seed, gg, dev)
            stats.append(check_sampled(a32[gg * max_m:(gg + 1) * max_m], qa[gg * max_m:(gg + 1) * max_m],
                                       sa[gg * max_m:(gg + 1) * max_m], b32, qb[gg], sb[gg], d[gg], rows,
                                       blocks, cols, f"decode[{idx}] group {gg}"))
    assert_exact_rate(stats, 0.95, f"decode[{idx}]")


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
