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


def _random_shapes(count, seed, m_lo=1, m_hi=700):
    """Seeded shapes within the documented contract: M from m_lo to m_hi
    (log-uniform), N a multiple of 8 up to 2400, K a multiple of 128 up to 5120."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        m = int(np.exp(rng.uniform(np.log(m_lo), np.log(m_hi))))
        n = 8 * int(rng.integers(1, 301))
        k = 128 * int(rng.integers(1, 41))
        out.append((max(m, 1), n, k))
    return out


@pytest.mark.parametrize("m,n,k", _random_shapes(16, seed=2024) + _random_shapes(6, seed=2025, m_lo=700, m_hi=3000)
                         + [(4096, 2880, 640), (3000, 4000, 1024)])   # 256x256 and 192x256 tiles
def test_dense_random_shapes_padded_strides(m, n, k):
    """Random shapes under the planner's own plan (split K included), with A and
    B rows padded past K, D rows padded past N and A's scales in either layout:
    every element matches the oracle, and no padding byte of D is written."""
    rng = np.random.default_rng(m * 131 + n * 7 + k)
    plan = dg.tile_config(m, n, k)
    print(f"random dense {m}x{n}x{k} plan {plan}", flush=True)
    qa, sa, qb, sb = _host_problem(m, n, k, seed=int(rng.integers(1 << 30)))
    pad_a, pad_b, pad_d = (16 * int(rng.integers(0, 5)) for _ in range(3))
    a_buf = torch.zeros((m, k + pad_a), dtype=torch.uint8, device=device())
    a_buf[:, :k] = torch.from_numpy(qa).to(device())
    b_buf = torch.zeros((n, k + pad_b), dtype=torch.uint8, device=device())
    b_buf[:, :k] = torch.from_numpy(qb).to(device())
    d_buf = sentinel_like((m, n + pad_d))
    sa_t = upload(np.ascontiguousarray(sa.T)).t() if rng.integers(2) else upload(sa)
    dg.fp8_gemm_nt((a_buf[:, :k].view(torch.float8_e4m3fn), sa_t), (b_buf[:, :k].view(torch.float8_e4m3fn),
                                                                    upload(sb)), d_buf[:, :n])
    torch.cuda.synchronize()
    got = bits(d_buf)
    assert np.all(got[:, n:] == 0x7FC1), "padding columns of D were written"
    assert_gemm_close(got[:, :n], ogemm.gemm_nt(qa, sa, qb, sb), f"random {m}x{n}x{k} plan {plan}")


@pytest.mark.parametrize("m,n,k", [(64, 264, 65536), (300, 136, 32768)])
def test_dense_long_k(m, n, k):
    # 512 and 256 K blocks: the per-block mantissa rescale runs hundreds of
    # times per accumulator, over the split-K plan the planner picks (M = 64)
    # and over whole tiles (M = 300), and with no workspace (no split)
    print(f"dense long K {m}x{n}x{k} plan {dg.tile_config(m, n, k)}", flush=True)
    qa, sa, qb, sb = _host_problem(m, n, k, seed=m + k)
    want = ogemm.gemm_nt(qa, sa, qb, sb)
    assert_gemm_close(_gpu_dense(qa, sa, qb, sb), want, f"{m}x{n}x{k}")
    a, b = (upload_codes(qa), upload(sa)), (upload_codes(qb), upload(sb))
    d = sentinel_like((m, n))
    dg.fp8_gemm_nt(a, b, d, workspace=None)
    torch.cuda.synchronize()
    assert_gemm_close(bits(d), want, f"{m}x{n}x{k} unsplit")


# plans: 128x128 tiles, 64x64 tiles, 256x256 tiles (A side, B side), 64x64 tiles split 4 ways over K
@pytest.mark.parametrize("m,n,k,side", [(4095, 1024, 512, "a"), (64, 4088, 512, "b"), (1000, 4088, 256, "b"),
                                        (4095, 4096, 2048, "a"), (4088, 4088, 1024, "b"), (64, 4088, 7168, "b")])
def test_dense_operand_offsets_near_the_32bit_limit(m, n, k, side):
    """The kernels address operand rows with 32-bit per-lane byte offsets (rows x
    leading dimension < 2^32).  With rows 1 MiB apart, the last rows of A (or B)
    lie just under 4 GiB from the first: every output still matches the oracle,
    and a problem one row (A) or eight rows (B) larger is rejected before any
    launch, leaving D untouched."""
    ld = 1 << 20
    rows = m if side == "a" else n
    more = 1 if side == "a" else 8
    assert (rows - 1) * ld + k < 2 ** 32 <= (rows + more) * ld
    print(f"dense {m}x{n}x{k}, {side} rows {ld} bytes apart, plan {dg.tile_config(m, n, k)}", flush=True)
    qa, sa, qb, sb = _host_problem(m, n, k, seed=m + n + k)
    dev = device()
    buf = torch.zeros((rows + more - 1) * ld + k, dtype=torch.uint8, device=dev)

    def spread(r, q=None):
        v = buf.as_strided((r, k), (ld, 1))
        if q is not None:
            v.copy_(torch.from_numpy(q).to(dev))
        return v.view(torch.float8_e4m3fn)

    if side == "a":
        a, b = (spread(m, qa), upload(sa)), (upload_codes(qb), upload(sb))
    else:
        a, b = (upload_codes(qa), upload(sa)), (spread(n, qb), upload(sb))
    d = sentinel_like((m, n))
    dg.fp8_gemm_nt(a, b, d)
    torch.cuda.synchronize()
    assert_gemm_close(bits(d), ogemm.gemm_nt(qa, sa, qb, sb), f"{m}x{n}x{k} {side} at the offset limit")
    # one row more no longer fits the 32-bit offsets
    if side == "a":
        a = (spread(m + more), upload(np.ones((m + more, k // 128), np.float32)))
        d = sentinel_like((m + more, n))
    else:
        b = (spread(n + more), upload(np.ones(((n + more + 127) // 128, k // 128), np.float32)))
        d = sentinel_like((m, n + more))
    with pytest.raises(dg.DgError) as err:
        dg.fp8_gemm_nt(a, b, d)
    assert err.value.status == dg.DG_ERROR_NOT_SUPPORTED
    torch.cuda.synchronize()
    assert bool((d.view(torch.int16) == 0x7FC1).all()), "a rejected call wrote D"


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


@pytest.mark.parametrize("m,n,k,ue8m0", [(300, 520, 640, True), (64, 2112, 1536, True), (4096, 2880, 640, True),
                                         (300, 520, 128, False), (4096, 2880, 128, False)])
def test_negation_and_zero_rows_bit_exact(m, n, k, ue8m0):
    """Sign symmetry of the whole path, bit for bit, under the planner's own plan
    (128x64 tiles, split K and 256x256 tiles among the shapes): negating A (or B)
    negates every nonzero output, a zero stays a zero, and A rows of zero codes
    give rows of +0.  This holds wherever no K block's promotion drops low bits
    of the running fp32 sum: over a single K block, and on these inputs with
    power-of-two scales, whose running sums keep few bits (they add up products
    the MFMA has already cut to its 14-bit window, with no rescale).  With fp32
    scales over several K blocks the rescaled running sum carries all 24 bits,
    the MFMA truncates the ones a larger block sum pushes below the result's
    grid toward minus infinity (pinned by test_gpu_accumulator.py's
    test_mfma_accumulator_input_alignment), and a few outputs in a million then
    differ from the exact negation by a bf16 ulp or two."""
    print(f"negation {m}x{n}x{k} ue8m0={ue8m0} plan {dg.tile_config(m, n, k)}", flush=True)
    qa, sa, qb, sb = _host_problem(m, n, k, seed=m + n + k, ue8m0=ue8m0)
    zero_rows = sorted({0, min(17, m - 1), m - 1})
    qa[zero_rows] = 0
    base = _gpu_dense(qa, sa, qb, sb)
    neg_a = _gpu_dense(qa ^ np.uint8(0x80), sa, qb, sb)
    neg_b = _gpu_dense(qa, sa, qb ^ np.uint8(0x80), sb)
    zero = (base & 0x7FFF) == 0
    assert np.all(base[zero_rows] == 0), "rows of zero codes are not +0"
    for got, what in ((neg_a, "-A"), (neg_b, "-B")):
        assert np.array_equal(got[~zero], base[~zero] ^ np.uint16(0x8000)), f"{what}: not the negation"
        assert np.all((got[zero] & 0x7FFF) == 0), f"{what}: a zero output is not a zero"
    assert_gemm_close(base, ogemm.gemm_nt(qa, sa, qb, sb), f"negation base {m}x{n}x{k}")


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


@pytest.mark.parametrize("m,n,k", [(300, 520, 640), (64, 520, 4096), (4096, 4096, 512)])
def test_zero_subnormal_and_nonfinite_scales(m, n, k):
    """A zero scale contributes nothing and a subnormal one its exact value (the
    plain definition); an infinite or NaN scale gives NaN in the rows (or the
    128-column block) it weights.  Covers the 128x64 / split-K / 256x256 tiles."""
    print(f"special scales {m}x{n}x{k} tile {dg.tile_config(m, n, k)}", flush=True)
    qa, sa, qb, sb = _host_problem(m, n, k, seed=m + n)
    sub = np.float32(2.0 ** -130)                   # subnormal fp32
    sb[:, 0] *= np.float32(2.0 ** 60)               # K block 0: products of sub with sb are normal
    sa[5, :] = 0.0                                  # whole row: exactly zero output
    sa[7, 2] = 0.0
    sa[9, 1] = -0.0
    sa[11, 3] = sub
    sa[12, :] = 0.0                                 # row 12: only a subnormal-scaled block contributes
    sa[12, 0] = -sub
    sb[1, 1] = 0.0                                  # B block of columns 128..255, K block 1
    sb[0, 3] = sub
    sa[13, 1] = np.inf                              # row 13: NaN
    sb[2, 2] = np.nan                               # columns 256..383: NaN
    got = _gpu_dense(qa, sa, qb, sb)
    sa_ref, sb_ref = sa.copy(), sb.copy()
    sa_ref[13, 1], sb_ref[2, 2] = 1.0, 1.0          # placeholders: those outputs are checked for NaN below
    want = ogemm.gemm_nt(qa, sa_ref, qb, sb_ref)
    f = (got.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isnan(f[13])) and np.all(np.isnan(f[:, 256:384]))
    keep_r = np.array([i for i in range(m) if i != 13])
    keep_c = np.array([j for j in range(n) if not 256 <= j < 384])
    assert np.all(f[5, keep_c] == 0.0), "a row whose scales are all zero must be exactly zero"
    assert np.any(f[12, keep_c] != 0.0)
    assert_gemm_close(got[12, keep_c], want[12, keep_c], "row weighted by a subnormal scale only")
    assert_gemm_close(got[np.ix_(keep_r, keep_c)], want[np.ix_(keep_r, keep_c)], f"special scales {m}x{n}x{k}")


def test_split_k_auto_workspace_on_two_concurrent_streams():
    """Split-K calls with the default workspace on two streams that overlap:
    each stream gets its own workspace, so neither corrupts the other's partial
    tiles or arrival counters."""
    shapes = [(64, 2112, 7168), (128, 7168, 2048)]
    for s in shapes:
        assert dg.tile_config(*s)[2] > 1, "shape no longer splits"
    probs = [_host_problem(m, n, k, seed=90 + i) for i, (m, n, k) in enumerate(shapes)]
    dev_in = [((upload_codes(qa), upload(sa)), (upload_codes(qb), upload(sb))) for qa, sa, qb, sb in probs]
    wants = [ogemm.gemm_nt(*p) for p in probs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rep in range(6):
        for i, st in enumerate(streams):
            j = (i + rep) % 2                               # both shapes on both streams
            (m, n, _) = shapes[j]
            with torch.cuda.stream(st):
                d = sentinel_like((m, n))
                dg.fp8_gemm_nt(dev_in[j][0], dev_in[j][1], d)
                outs.append((j, d))
    torch.cuda.synchronize()
    first = {}
    for j, d in outs:
        got = bits(d)
        if j not in first:
            assert_gemm_close(got, wants[j], f"stream split-K {shapes[j]}")
            first[j] = got
        assert np.array_equal(got, first[j]), f"{shapes[j]}: a concurrent call changed the result"


def test_binding_rejects_wrong_scale_shapes_before_launch():
    qa, sa, qb, sb = _host_problem(128, 264, 512, seed=3)
    a, b = upload_codes(qa), upload_codes(qb)
    d = sentinel_like((128, 264))
    with pytest.raises(ValueError):
        dg.fp8_gemm_nt((a, upload(sa[:, :3])), (b, upload(sb)), d)
    with pytest.raises(ValueError):
        dg.fp8_gemm_nt((a, upload(sa)), (b, upload(sb[:2])), d)
    torch.cuda.synchronize()
    assert bool((d.view(torch.int16) == 0x7FC1).all()), "output touched"


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


def check_sampled(a32, qa, sa, b32, qb, sb, d, rows, blocks, cols, what, ue8m0=False, min_exact=None):
    """Oracle re-quantization of the sampled pieces (bit-exact vs the GPU casts)
    and the sampled GEMM outputs (tolerance).  Returns the tolerance statistics
    and the counts of sampled outputs that equal the oracle's bf16 result bit for
    bit (``n_exact``) or lie more than one bf16 ulp from it (``n_far``), out of
    ``n``; with ``min_exact`` those rates are asserted here (assert_exact_rate)."""
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
    stats = assert_gemm_close(got, want, what)
    g, w = got.astype(np.int32), want.astype(np.int32)
    # distance in bf16 ulps between outputs of equal sign; a sign flip counts as far
    ulps = np.where((g & 0x8000) == (w & 0x8000), np.abs((g & 0x7FFF) - (w & 0x7FFF)), 1 << 16)
    stats.update(n=int(ulps.size), n_exact=int(np.sum(ulps == 0)), n_far=int(np.sum(ulps > 1)))
    if min_exact is not None:
        assert_exact_rate([stats], min_exact, what)
    return stats


def assert_exact_rate(stats, min_exact, what):
    """At least ``min_exact`` of the sampled outputs (summed over check_sampled
    results) equal the oracle's exactly rounded bf16 result bit for bit, and at
    most 1% lie more than one bf16 ulp away from it."""
    n = sum(s["n"] for s in stats)
    exact = sum(s["n_exact"] for s in stats) / n
    far = sum(s["n_far"] for s in stats) / n
    assert exact >= min_exact, f"{what}: only {exact:.4f} of {n} sampled outputs equal the oracle's bits"
    assert far <= 0.01, f"{what}: {far:.4f} of {n} sampled outputs are over one bf16 ulp away"


def mn_major_scales(rows, kblocks):
    """fp32 scale buffer [rows, kblocks] in the MN-major layout (element (r, kb)
    at kb * rows + r) that the casts write and the benchmark's GEMMs read."""
    return torch.empty((kblocks, rows), dtype=torch.float32, device=device()).t()


@pytest.mark.parametrize("idx", range(15))
def test_dense_full_size_sampled(idx):
    m, n, k = synth.config1_shapes()[idx]
    seed = synth.seed_for(1, idx)
    print(f"dense full size {m}x{n}x{k}", flush=True)
    dev = device()
    a32 = synth.draw_activation_device(m, k, seed, dev)
    b32 = synth.draw_weight_device(n, k, seed, 0, dev)
    qa, sa = dg.per_token_cast_fp8(a32, sf=mn_major_scales(m, k // 128))
    assert sa.stride() == (1, m)
    qb, sb = dg.per_block_cast_fp8(b32)
    d = sentinel_like((m, n))
    dg.fp8_gemm_nt((qa, sa), (qb, sb), d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    rows = sample_rows(rng, m, 24)
    blocks, cols = sample_blocks_and_cols(rng, n, 3, 12)
    # most outputs are the exactly rounded result: about 98.8% on these shapes (the
    # rest one bf16 ulp off, or near zero after cancellation)
    check_sampled(a32, qa, sa, b32, qb, sb, d, rows, blocks, cols, f"{m}x{n}x{k}", min_exact=0.95)
    # every output element was written (no sentinel left, nothing non-finite)
    assert bool(torch.isfinite(d.float()).all())


def test_dense_full_size_every_element():
    """4096 x 4096 x 7168 as the benchmark runs it (MN-major A scales from the
    cast, 256x256 tiles): every output element against the oracle, which
    re-quantizes the whole fp32 operands (its codes and scales must equal the
    GPU casts' bit for bit)."""
    m, n, k = 4096, 4096, 7168
    idx = synth.config1_shapes().index((m, n, k))
    seed = synth.seed_for(1, idx)
    assert dg.tile_config(m, n, k) == (256, 256, 1)
    dev = device()
    a32 = synth.draw_activation_device(m, k, seed, dev)
    b32 = synth.draw_weight_device(n, k, seed, 0, dev)
    qa, sa = dg.per_token_cast_fp8(a32, sf=mn_major_scales(m, k // 128))
    qb, sb = dg.per_block_cast_fp8(b32)
    d = sentinel_like((m, n))
    dg.fp8_gemm_nt((qa, sa), (qb, sb), d)
    torch.cuda.synchronize()
    got = bits(d)
    oqa, osa = quant.per_token_cast(a32.cpu().numpy())
    oqb, osb = quant.per_block_cast(b32.cpu().numpy())
    assert np.array_equal(codes(qa), oqa) and np.array_equal(sa.cpu().numpy().view(np.uint32), osa.view(np.uint32))
    assert np.array_equal(codes(qb), oqb) and np.array_equal(sb.cpu().numpy().view(np.uint32), osb.view(np.uint32))
    print("oracle casts agree; computing the full reference", flush=True)
    want = ogemm.gemm_nt(oqa, osa, oqb, osb)
    stats = assert_gemm_close(got, want, f"{m}x{n}x{k} every element")
    print(f"every element within tolerance, rel. Frobenius {stats['fro']:.2e}", flush=True)


def test_dense_step_graph_replays_bit_for_bit():
    """The benchmark's dense step (the 15 LLM-layer GEMMs at full size, the
    planner's own plans, split-K shapes on their own workspaces) captured once in
    a HIP graph and replayed three times, with eager calls on the same
    workspaces in between: every replay gives the eager step's bits."""
    dev = device()
    shapes = synth.config1_shapes()
    probs = []
    for idx, (m, n, k) in enumerate(shapes):
        g = torch.Generator(device=dev).manual_seed(synth.seed_for(1, idx))
        qa = (torch.randint(0, 0x7F, (m, k), dtype=torch.uint8, device=dev, generator=g)
              | (torch.randint(0, 2, (m, k), dtype=torch.uint8, device=dev, generator=g) << 7))
        qb = (torch.randint(0, 0x7F, (n, k), dtype=torch.uint8, device=dev, generator=g)
              | (torch.randint(0, 2, (n, k), dtype=torch.uint8, device=dev, generator=g) << 7))
        sa = mn_major_scales(m, k // 128)
        sa.copy_(torch.exp2(torch.rand((m, k // 128), device=dev, generator=g) * 8 - 12))
        sb = torch.exp2(torch.rand(((n + 127) // 128, k // 128), device=dev, generator=g) * 8 - 12)
        ws = torch.zeros(max(dg.workspace_size(m, n, k), 16), dtype=torch.uint8, device=dev)
        probs.append(((qa.view(torch.float8_e4m3fn), sa), (qb.view(torch.float8_e4m3fn), sb), ws))

    def step(outs):
        for (a, b, ws), d in zip(probs, outs):
            dg.fp8_gemm_nt(a, b, d, workspace=ws)

    eager = [sentinel_like((a[0].shape[0], b[0].shape[0])) for a, b, _ in probs]
    step(eager)
    torch.cuda.synchronize()
    want = [bits(d) for d in eager]
    outs = [sentinel_like(d.shape) for d in eager]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    print("dense step: capturing 15 GEMMs", flush=True)
    with torch.cuda.graph(graph, stream=s):
        step(outs)
    torch.cuda.synchronize()
    for r in range(3):
        for d in outs:
            d.view(torch.int16).fill_(0x7FC1)
        print(f"dense step: replay {r}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        for (m, n, k), d, w in zip(shapes, outs, want):
            assert np.array_equal(bits(d), w), f"replay {r}, {m}x{n}x{k}: differs from the eager step"
        step(eager)                      # eager calls on the same workspaces between replays
        torch.cuda.synchronize()
        for (m, n, k), d, w in zip(shapes, eager, want):
            assert np.array_equal(bits(d), w), f"eager after replay {r}, {m}x{n}x{k}"
    del graph
