"""Every dense kernel instance, with and without the cross-workgroup split-K,
against the CPU oracle.

The cost model picks one (instance, split) plan per shape, so most plans never
run on the shapes the other tests use.  Here every case forces the plan through
dg_set_dense_plan:

* ragged M and N (tails inside a tile) and K of 1 to 25 blocks, so that split
  ranges end short and some splits get a single K block;
* fp32 scales (MN-major A scales as the benchmark uses) and packed UE8M0 words
  (bit-identical to the fp32 path on power-of-two scales);
* the fp32 addend C, a persistent grid narrower than the unit count (several
  units per workgroup), determinism, and the split count's independence of the
  grid width.
Element-wise acceptance as in gpu_util (the oracle is fp64 with bf16 output).
"""
import contextlib

import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm
from oracle import quant, ue8m0
from gpu_util import assert_gemm_close, bits, sentinel_like, upload, upload_codes

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_fp8_gemm_amd as dg  # noqa: E402

LARGE, MID, HUGE, SKINNY128, SKINNY64, TALL = 0, 1, 2, 3, 4, 6
TILES = {LARGE: (128, 256), MID: (128, 128), HUGE: (256, 256), SKINNY128: (128, 64), SKINNY64: (64, 64),
         TALL: (192, 256)}
SPLIT_K = [LARGE, MID, SKINNY128, SKINNY64]          # instances with a split-K variant


@contextlib.contextmanager
def forced_plan(inst, splits):
    dg.set_dense_plan(inst, splits)
    try:
        yield
    finally:
        dg.set_dense_plan(-1)


def _problem(m, n, k, seed, ue8m0_scales=False):
    w = synth.dense(m, n, k, seed)
    qa, sa = quant.per_token_cast(w.a, ue8m0_scales)
    qb, sb = quant.per_block_cast(w.b, ue8m0_scales)
    return qa, sa, qb, sb


def _mn_major(sf):
    return upload(np.ascontiguousarray(sf.T)).t()


def _run(qa, sa_t, qb, sb_t, c=None):
    d = sentinel_like((qa.shape[0], qb.shape[0]))
    dg.fp8_gemm_nt((upload_codes(qa), sa_t), (upload_codes(qb), sb_t), d, c=c)
    torch.cuda.synchronize()
    return bits(d)


def _splits(k, splits):
    # the plan's K split: blocks per split rounded up, empty splits dropped
    kb = k // 128
    s = min(splits, kb)
    per = -(-kb // s)
    return -(-kb // per)


CASES = [(1, 8, 128), (37, 264, 640), (64, 2112, 768), (100, 520, 1408), (128, 136, 1920),
         (200, 392, 512), (64, 1032, 3200)]


def _plans():
    return [(i, s) for i in SPLIT_K for s in (1, 2, 5)] + [(HUGE, 1), (TALL, 1)]


@pytest.mark.parametrize("inst,splits", _plans())
@pytest.mark.parametrize("m,n,k", CASES)
def test_forced_plan_parity(m, n, k, inst, splits):
    with forced_plan(inst, splits):
        bm, bn, sp = dg.tile_config(m, n, k)
        assert (bm, bn) == TILES[inst] and sp == _splits(k, splits)
        print(f"forced plan {m}x{n}x{k} instance {inst} splits {sp}", flush=True)
        qa, sa, qb, sb = _problem(m, n, k, seed=m * 5 + n + k + inst)
        got = _run(qa, _mn_major(sa), qb, upload(sb))
    assert_gemm_close(got, ogemm.gemm_nt(qa, sa, qb, sb), f"{m}x{n}x{k} inst {inst} splits {sp}")


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("inst", SPLIT_K)
@pytest.mark.parametrize("m,n,k", [(37, 264, 640), (128, 1032, 3200)])
def test_forced_plan_packed_equals_fp32_path(m, n, k, inst, splits):
    print(f"forced plan ue8m0 {m}x{n}x{k} instance {inst} splits {splits}", flush=True)
    qa, sa, qb, sb = _problem(m, n, k, seed=m + n + k, ue8m0_scales=True)
    pack = lambda sf: dg.pack_ue8m0(upload(sf))  # noqa: E731
    with forced_plan(inst, splits):
        ref = _run(qa, _mn_major(sa), qb, upload(sb))
        got = _run(qa, pack(sa), qb, pack(sb))
    assert np.array_equal(got, ref)
    want = ogemm.gemm_nt(qa, ue8m0.unpack(ue8m0.pack(sa), sa.shape[1]), qb, ue8m0.unpack(ue8m0.pack(sb), sb.shape[1]))
    assert_gemm_close(got, want, f"packed {m}x{n}x{k} inst {inst}")


@pytest.mark.parametrize("inst,splits", [(SKINNY64, 1), (SKINNY64, 4), (SKINNY128, 3), (MID, 2), (LARGE, 5),
                                         (HUGE, 1), (TALL, 1)])
def test_forced_plan_addend(inst, splits):
    m, n, k = 100, 520, 2048
    qa, sa, qb, sb = _problem(m, n, k, seed=11)
    c = (np.random.default_rng(12).standard_normal((m, n)) * 4).astype(np.float32)
    with forced_plan(inst, splits):
        print(f"forced plan addend instance {inst} splits {splits}", flush=True)
        got = _run(qa, _mn_major(sa), qb, upload(sb), c=upload(c))
    assert_gemm_close(got, ogemm.gemm_nt(qa, sa, qb, sb, c), f"addend inst {inst} splits {splits}")


@pytest.mark.parametrize("inst,splits", [(SKINNY64, 6), (SKINNY128, 4), (MID, 3), (LARGE, 2), (HUGE, 1)])
def test_forced_plan_narrow_grid_same_bits(inst, splits):
    # 3 workgroups walk all units in turn; the result must not change
    m, n, k = 96, 1032, 3072
    qa, sa, qb, sb = _problem(m, n, k, seed=13)
    with forced_plan(inst, splits):
        print(f"forced plan narrow grid instance {inst} splits {splits}", flush=True)
        ref = _run(qa, _mn_major(sa), qb, upload(sb))
        again = _run(qa, _mn_major(sa), qb, upload(sb))
        try:
            dg.set_num_cus(3)
            narrow = _run(qa, _mn_major(sa), qb, upload(sb))
        finally:
            dg.set_num_cus(0)
    assert np.array_equal(ref, again)
    assert np.array_equal(ref, narrow)
    assert_gemm_close(ref, ogemm.gemm_nt(qa, sa, qb, sb), f"narrow grid inst {inst}")
