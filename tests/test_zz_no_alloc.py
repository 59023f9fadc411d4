"""The dense GEMM entry point that allocates nothing (dg_fp8_gemm_nt_noalloc),
called through the C ABI, against the workspace entry point it stands in for
(dg_fp8_gemm_nt_ws with a workspace of the planned size) and the oracle.

Two split-K calls in a row on the library's static scratch, the second one on
a smaller problem, then an unsplit one; each must give the workspace entry
point's bits (same plan, same kernels) and pass the oracle tolerance.  A
problem whose split plan needs more scratch than the static maximum is
rejected before anything is launched.  Split-K calls captured in a HIP graph
replay with the eager calls' bits.
"""
import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm
from oracle import quant
from gpu_util import assert_gemm_close, bits, device, sentinel_like, upload, upload_codes

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_fp8_gemm_amd as dg  # noqa: E402

SCRATCH_BYTES = (256 << 10) + (16 << 20)


def _problem(m, n, k, seed):
    w = synth.dense(m, n, k, seed)
    qa, sa = quant.per_token_cast(w.a)
    qb, sb = quant.per_block_cast(w.b)
    return qa, sa, qb, sb


def _args(a, sa, b, sb, d):
    m, k = a.shape
    n = b.shape[0]
    return (a.data_ptr(), a.stride(0), sa.data_ptr(), sa.stride(0), sa.stride(1), b.data_ptr(), b.stride(0),
            sb.data_ptr(), sb.stride(0), sb.stride(1), d.data_ptr(), d.stride(0), m, n, k)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("shapes", [[(128, 7168, 2048), (64, 2112, 7168), (300, 520, 640)]])
def test_noalloc_matches_the_workspace_entry_point(shapes):
    outs = []
    for i, (m, n, k) in enumerate(shapes):
        need = dg.workspace_size(m, n, k)
        assert need <= SCRATCH_BYTES
        print(f"no-alloc {m}x{n}x{k}: workspace {need} bytes, plan {dg.tile_config(m, n, k)}", flush=True)
        qa, sa, qb, sb = _problem(m, n, k, seed=70 + i)
        a, b, sa_t, sb_t = upload_codes(qa), upload_codes(qb), upload(sa), upload(sb)
        d = sentinel_like((m, n))
        st = dg.lib.dg_fp8_gemm_nt_noalloc(*_args(a, sa_t, b, sb_t, d), _stream())
        assert st == dg.DG_SUCCESS, dg.lib.dg_status_string(st)
        outs.append((d, (a, sa_t, b, sb_t), (qa, sa, qb, sb), need))
    torch.cuda.synchronize()     # the calls ran back to back on one stream, sharing the scratch
    for d, (a, sa_t, b, sb_t), host, need in outs:
        m, n = d.shape
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=device())
        d_ws = sentinel_like((m, n))
        st = dg.lib.dg_fp8_gemm_nt_ws(*_args(a, sa_t, b, sb_t, d_ws), ctypes.c_void_p(ws.data_ptr()),
                                      ctypes.c_size_t(ws.numel()), _stream())
        assert st == dg.DG_SUCCESS
        torch.cuda.synchronize()
        got = bits(d)
        assert np.array_equal(got, bits(d_ws)), f"{m}x{n}: differs from the workspace entry point"
        assert_gemm_close(got, ogemm.gemm_nt(*host), f"no-alloc {m}x{n}")


def test_noalloc_rejects_plans_beyond_the_static_scratch():
    m, n, k = 512, 3072, 32768
    need = dg.workspace_size(m, n, k)
    assert need > SCRATCH_BYTES, "shape no longer needs more than the static scratch"
    dev = device()
    a = torch.zeros((m, k), dtype=torch.uint8, device=dev)
    b = torch.zeros((n, k), dtype=torch.uint8, device=dev)
    sa = torch.ones((m, k // 128), dtype=torch.float32, device=dev)
    sb = torch.ones((n // 128, k // 128), dtype=torch.float32, device=dev)
    d = sentinel_like((m, n))
    st = dg.lib.dg_fp8_gemm_nt_noalloc(*_args(a, sa, b, sb, d), _stream())
    assert st == dg.DG_ERROR_SCRATCH_LIMIT
    with pytest.raises(dg.DgError):
        dg.fp8_gemm_nt_noalloc((a, sa), (b, sb), d)
    torch.cuda.synchronize()
    assert bool((d.view(torch.int16) == 0x7FC1).all()), "output touched"


def test_noalloc_under_graph_capture():
    """What the entry point is for: split-K calls on the static scratch recorded
    in a HIP graph (no allocation may happen while capturing), replayed three
    times with eager calls on the same scratch in between.  Every replay must
    give the bits of the eager calls."""
    shapes = [(128, 7168, 2048), (64, 2112, 7168)]
    probs = []
    for i, (m, n, k) in enumerate(shapes):
        assert dg.tile_config(m, n, k)[2] > 1, "shape no longer splits K"
        qa, sa, qb, sb = _problem(m, n, k, seed=90 + i)
        probs.append((upload_codes(qa), upload(sa), upload_codes(qb), upload(sb)))
    want = []
    for a, sa_t, b, sb_t in probs:
        d = sentinel_like((a.shape[0], b.shape[0]))
        dg.fp8_gemm_nt_noalloc((a, sa_t), (b, sb_t), d)
        want.append(d)
    torch.cuda.synchronize()
    want_bits = [bits(d) for d in want]
    outs = [sentinel_like(d.shape) for d in want]
    side = sentinel_like(want[0].shape)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    print("no-alloc: capturing two split-K calls", flush=True)
    with torch.cuda.graph(g, stream=s):
        for (a, sa_t, b, sb_t), d in zip(probs, outs):
            dg.fp8_gemm_nt_noalloc((a, sa_t), (b, sb_t), d)
    torch.cuda.synchronize()
    for r in range(3):
        for d in outs:
            d.view(torch.int16).fill_(0x7FC1)
        print(f"no-alloc: replay {r}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        for d, wb, (m, n, k) in zip(outs, want_bits, shapes):
            assert np.array_equal(bits(d), wb), f"replay {r}, {m}x{n}x{k}: differs from the eager call"
        # an eager call between replays shares the scratch (its counters must come back zero)
        a, sa_t, b, sb_t = probs[0]
        dg.fp8_gemm_nt_noalloc((a, sa_t), (b, sb_t), side)
        torch.cuda.synchronize()
        assert np.array_equal(bits(side), want_bits[0])
    del g
