"""Packed UE8M0 scales on the GPU: the pack kernel and the packed-scale GEMMs.

* dg_pack_ue8m0 against the oracle's packing, bit for bit: power-of-two and
  arbitrary positive scales, K-block counts of every residue mod 4, strided
  (MN-major) inputs and outputs.
* The packed-scale GEMMs (dense, split-K, contiguous, masked) against the
  fp32-scale GEMMs on the same power-of-two scales: the two must agree bit for
  bit (with power-of-two scales the fp32 path's rescale factors are exactly 1),
  and against the oracle evaluated on the unpacked scales.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm
from oracle import quant, ue8m0
from gpu_util import SENTINEL, assert_gemm_close, bits, sentinel_like, upload, upload_codes

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_fp8_gemm_amd as dg  # noqa: E402


def _pack(sf: np.ndarray) -> torch.Tensor:
    return dg.pack_ue8m0(upload(np.ascontiguousarray(sf, dtype=np.float32)))


@pytest.mark.parametrize("rows,kblocks", [(1, 1), (7, 5), (300, 56), (129, 3), (64, 2), (33, 12)])
def test_pack_kernel_matches_oracle(rows, kblocks):
    rng = np.random.default_rng(rows * 100 + kblocks)
    pow2 = (np.float32(2.0) ** rng.integers(-40, 20, size=(rows, kblocks)).astype(np.float32)).astype(np.float32)
    other = (2.0 ** rng.uniform(-40, 20, size=(rows, kblocks))).astype(np.float32)
    for sf in (pow2, other):
        got = _pack(sf)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), ue8m0.pack(sf))


def test_pack_kernel_strided_layouts():
    rng = np.random.default_rng(3)
    sf = (np.float32(2.0) ** rng.integers(-30, 5, size=(200, 9)).astype(np.float32)).astype(np.float32)
    src = upload(np.ascontiguousarray(sf.T)).t()                       # MN-major input, strides (1, 200)
    out = torch.zeros((3, 200), dtype=torch.int32, device=src.device).t()   # MN-major output
    dg.pack_ue8m0(src, out=out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ue8m0.pack(sf))


def _dense_pow2(m, n, k, seed):
    w = synth.dense(m, n, k, seed)
    qa, sa = quant.per_token_cast(w.a, True)
    qb, sb = quant.per_block_cast(w.b, True)
    return qa, sa, qb, sb


def _run_dense(qa, sa_t, qb, sb_t):
    d = sentinel_like((qa.shape[0], qb.shape[0]))
    dg.fp8_gemm_nt((upload_codes(qa), sa_t), (upload_codes(qb), sb_t), d)
    torch.cuda.synchronize()
    return bits(d)


@pytest.mark.parametrize("m,n,k", [(128, 256, 512), (300, 520, 640), (129, 264, 1536), (1, 8, 128),
                                   (520, 392, 384), (256, 1024, 1152)])
def test_dense_packed_equals_fp32_path(m, n, k):
    print(f"dense ue8m0 {m}x{n}x{k}", flush=True)
    qa, sa, qb, sb = _dense_pow2(m, n, k, seed=m + n + k)
    ref = _run_dense(qa, upload(sa), qb, upload(sb))
    got = _run_dense(qa, _pack(sa), qb, _pack(sb))
    assert np.array_equal(got, ref)
    want = ogemm.gemm_nt(qa, ue8m0.unpack(ue8m0.pack(sa), sa.shape[1]), qb, ue8m0.unpack(ue8m0.pack(sb), sb.shape[1]))
    assert_gemm_close(got, want, f"packed {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(2600, 3104, 640), (700, 1032, 768)])
def test_dense_packed_chained_tiles(m, n, k):
    """Workgroups walking many tiles in turn: each tile's first scale byte is
    picked by its own block index (5 and 6 blocks per tile, not multiples of 4)."""
    qa, sa, qb, sb = _dense_pow2(m, n, k, seed=k)
    ref = _run_dense(qa, upload(sa), qb, upload(sb))
    try:
        for cus in (1, 3):
            dg.set_num_cus(cus)
            assert np.array_equal(_run_dense(qa, _pack(sa), qb, _pack(sb)), ref), cus
    finally:
        dg.set_num_cus(0)


def test_dense_packed_mn_major_scale_words():
    qa, sa, qb, sb = _dense_pow2(300, 264, 1664, seed=9)          # 13 K blocks: a partial last word
    words = ue8m0.pack(sa)
    mn = upload(np.ascontiguousarray(words.T)).t()
    assert np.array_equal(_run_dense(qa, mn, qb, _pack(sb)), _run_dense(qa, upload(words), qb, _pack(sb)))


@pytest.mark.parametrize("m,n,k", [(64, 520, 4096), (16, 1536, 2048), (77, 136, 1280)])
def test_dense_packed_split_k_equals_fp32_path(m, n, k):
    assert dg.tile_config(m, n, k)[2] > 1, "shape no longer splits"
    print(f"split-K ue8m0 {m}x{n}x{k}", flush=True)
    qa, sa, qb, sb = _dense_pow2(m, n, k, seed=m * 3 + n)
    assert np.array_equal(_run_dense(qa, _pack(sa), qb, _pack(sb)), _run_dense(qa, upload(sa), qb, upload(sb)))


def test_contiguous_packed_equals_fp32_path():
    w = synth.contiguous(4, 700, [0.25] * 4, 392, 640, seed=31)
    qa, sa = quant.per_token_cast(w.a, True)
    pairs = [quant.per_block_cast(w.b[g], True) for g in range(4)]
    qb, sb = np.stack([p[0] for p in pairs]), np.stack([p[1] for p in pairs])
    out = []
    for sa_t, sb_t in ((upload(sa), upload(sb)), (_pack(sa), _pack(sb))):
        d = sentinel_like((qa.shape[0], qb.shape[1]))
        dg.m_grouped_fp8_gemm_nt_contiguous((upload_codes(qa), sa_t), (upload_codes(qb), sb_t), d,
                                            upload(w.m_indices))
        torch.cuda.synchronize()
        out.append(bits(d))
    assert np.array_equal(out[0], out[1])
    pad = w.m_indices < 0
    assert np.all(out[1][pad] == SENTINEL)
    want = ogemm.m_grouped_contiguous(qa, sa, qb, sb, w.m_indices)
    assert_gemm_close(out[1][~pad], want[~pad], "contiguous packed")


def test_masked_packed_equals_fp32_path():
    g, max_m, n, k = 5, 200, 264, 640
    masked_m = np.array([0, 1, 128, 200, 77], np.int32)
    w = synth.masked(g, max_m, n, k, 41, expected_m=100)
    qa, sa = quant.per_token_cast(w.a.reshape(g * max_m, k), True)
    qa, sa = qa.reshape(g, max_m, k), sa.reshape(g, max_m, k // 128)
    pairs = [quant.per_block_cast(w.b[i], True) for i in range(g)]
    qb, sb = np.stack([p[0] for p in pairs]), np.stack([p[1] for p in pairs])
    out = []
    # expected_m 100 runs 256-row tiles, 16 the 64-row decode tiles: same bits
    for sa_t, sb_t, hint in ((upload(sa), upload(sb), 100), (_pack(sa), _pack(sb), 100), (_pack(sa), _pack(sb), 16)):
        d = sentinel_like((g, max_m, n))
        dg.m_grouped_fp8_gemm_nt_masked((upload_codes(qa), sa_t), (upload_codes(qb), sb_t), d, upload(masked_m), hint)
        torch.cuda.synchronize()
        out.append(bits(d))
    assert np.array_equal(out[0], out[1])
    assert np.array_equal(out[1], out[2])
    want = ogemm.m_grouped_masked(qa, sa, qb, sb, masked_m)
    for i, c in enumerate(masked_m):
        assert np.all(out[1][i, c:] == SENTINEL)
        if c:
            assert_gemm_close(out[1][i, :c], want[i, :c], f"masked packed group {i}")


def test_dense_packed_256x256_tiles_mn_major_words():
    """The instance the benchmark times with packed scales: 256x256 tiles, A
    scale words in the MN-major layout.  Same bits as the fp32-scale path on the
    same power-of-two scales, and every element against the oracle."""
    m, n, k = 4096, 4096, 1536
    assert dg.tile_config(m, n, k) == (256, 256, 1)
    print(f"dense ue8m0 256x256 tiles {m}x{n}x{k}", flush=True)
    qa, sa, qb, sb = _dense_pow2(m, n, k, seed=17)
    words = ue8m0.pack(sa)
    packed = _run_dense(qa, upload(np.ascontiguousarray(words.T)).t(), qb, _pack(sb))
    fp32 = _run_dense(qa, upload(np.ascontiguousarray(sa.T)).t(), qb, upload(sb))
    assert np.array_equal(packed, fp32)
    assert_gemm_close(packed, ogemm.gemm_nt(qa, sa, qb, sb), f"packed 256x256 {m}x{n}x{k}")


def test_mixed_scale_formats_rejected():
    qa, sa, qb, sb = _dense_pow2(128, 256, 512, seed=1)
    d = sentinel_like((128, 256))
    with pytest.raises(TypeError):
        dg.fp8_gemm_nt((upload_codes(qa), _pack(sa)), (upload_codes(qb), upload(sb)), d)
