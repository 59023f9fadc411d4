"""The C-ABI library loads without a GPU, exports every function include/dgfp8.h
declares, and its host-side validation returns the documented status codes.
None of these calls reaches a kernel launch or any HIP runtime call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dgfp8.h")
LIB = os.path.join(ROOT, "moe_fp8_gemm_amd", "libdgfp8.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libdgfp8.so not built (run python moe_fp8_gemm_amd/build.py)")
    return ctypes.CDLL(LIB)


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("dg_fp8_gemm_nt", "dg_m_grouped_fp8_gemm_nt_contiguous", "dg_m_grouped_fp8_gemm_nt_masked",
                     "dg_per_token_cast_fp8", "dg_get_mk_alignment_for_contiguous_layout", "dg_set_num_cus",
                     "dg_get_num_cus", "dg_status_string"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_names_match_header():
    import moe_fp8_gemm_amd as m
    assert sorted(m._SIGNATURES) == _declared()


def test_status_strings_and_constants(lib):
    lib.dg_status_string.restype = ctypes.c_char_p
    assert lib.dg_status_string(0) == b"DG_SUCCESS"
    assert lib.dg_status_string(3) == b"DG_ERROR_MISALIGNED_LAYOUT"
    assert lib.dg_status_string(5) == b"DG_ERROR_SCRATCH_LIMIT"
    assert lib.dg_get_mk_alignment_for_contiguous_layout() == 128


# Fake, never-dereferenced, 256-aligned addresses: validation must reject the
# call before anything touches them.
P = ctypes.c_void_p(0x10000)


def _gemm(lib, a=P, lda=512, sfa=P, sfa_sm=4, sfa_sk=1, b=P, ldb=512, sfb=P, sfb_sn=4, sfb_sk=1,
          d=P, ldd=256, m=128, n=256, k=512):
    f = lib.dg_fp8_gemm_nt
    i = ctypes.c_int64
    return f(a, i(lda), sfa, i(sfa_sm), i(sfa_sk), b, i(ldb), sfb, i(sfb_sn), i(sfb_sk), d, i(ldd),
             i(m), i(n), i(k), None)


def test_dense_validation(lib):
    assert _gemm(lib, a=None) == 1                       # null -> INVALID_VALUE
    assert _gemm(lib, m=-1) == 1
    assert _gemm(lib, lda=256) == 1                      # lda < k
    assert _gemm(lib, sfa_sk=-1) == 1
    assert _gemm(lib, k=384 + 64, lda=512, ldb=512) == 2  # k % 128 -> NOT_SUPPORTED
    assert _gemm(lib, n=252, ldd=256) == 2               # n % 8
    assert _gemm(lib, lda=520) == 2                      # lda % 16
    assert _gemm(lib, a=ctypes.c_void_p(0x10008)) == 2   # misaligned A
    assert _gemm(lib, m=0) == 0                          # empty problem: success, no launch
    assert _gemm(lib, n=0) == 0
    assert _gemm(lib, m=0, k=0) == 0                     # empty before any other check
    assert _gemm(lib, k=0, lda=0, ldb=0) == 2            # empty sum over K: not supported


def test_dense_rejects_row_offsets_beyond_32_bits(lib):
    # The kernels address operand rows with 32-bit byte offsets from the operand
    # base: rows * ld must stay below 2^32 (these calls fail before any launch).
    k = 65536
    assert _gemm(lib, m=65536, k=k, lda=k, ldb=k, sfa_sm=k // 128, sfb_sn=k // 128) == 2
    assert _gemm(lib, n=65536, ldd=65536, k=k, lda=k, ldb=k, sfa_sm=k // 128, sfb_sn=k // 128) == 2


def test_workspace_entry_validation_and_size(lib):
    i = ctypes.c_int64
    f = lib.dg_fp8_gemm_nt_ws
    f.argtypes = [ctypes.c_void_p, i, ctypes.c_void_p, i, i, ctypes.c_void_p, i, ctypes.c_void_p, i, i,
                  ctypes.c_void_p, i, i, i, i, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]

    def call(ws, ws_bytes, **kw):
        a = dict(lda=512, sfa_sm=4, sfa_sk=1, ldb=512, sfb_sn=4, sfb_sk=1, ldd=256, m=128, n=256, k=512, a=P)
        a.update(kw)
        return f(a["a"], a["lda"], P, a["sfa_sm"], a["sfa_sk"], P, a["ldb"], P, a["sfb_sn"], a["sfb_sk"], P,
                 a["ldd"], a["m"], a["n"], a["k"], ws, ws_bytes, None)

    assert call(ctypes.c_void_p(0x10008), 1 << 20) == 2     # workspace not 16-byte aligned
    assert call(None, 0, a=None) == 1                        # validation as in dg_fp8_gemm_nt
    assert call(P, 1 << 20, m=0) == 0                        # empty problem
    size = lib.dg_fp8_gemm_nt_workspace_size
    size.restype = ctypes.c_size_t
    size.argtypes = [i, i, i]
    assert size(4096, 4096, 7168) == 0                       # enough tiles: never split
    assert size(64, 2112, 7168) > 256 * 1024                 # counter block + partial tiles
    assert size(0, 2112, 7168) == 0 and size(64, 2112, 7000) == 0


def test_contiguous_validation(lib):
    f = lib.dg_m_grouped_fp8_gemm_nt_contiguous
    i = ctypes.c_int64

    def call(m_total=256, groups=2, m_idx=P, n=256, k=512, ld=512):
        kb = ld // 128
        return f(P, i(ld), P, i(kb), i(1), P, i(ld), i(256 * ld), P, i(kb), i(1), i(2 * kb), P, i(256),
                 m_idx, i(m_total), i(n), i(k), ctypes.c_int(groups), None)

    assert call(m_total=200) == 3                        # MISALIGNED_LAYOUT
    assert call(groups=0) == 1
    assert call(m_idx=None) == 1
    assert call(k=500) == 2
    assert call(m_total=0) == 0
    assert call(m_total=65536, k=65536, ld=65536) == 2   # A row offsets beyond 32 bits


def test_contiguous_workspace_entry_validation(lib):
    f = lib.dg_m_grouped_fp8_gemm_nt_contiguous_ws
    i = ctypes.c_int64

    def call(ws, ws_bytes, m_total=256, groups=2, k=512, ld=512):
        kb = ld // 128
        return f(P, i(ld), P, i(kb), i(1), P, i(ld), i(256 * ld), P, i(kb), i(1), i(2 * kb), P, i(256),
                 P, i(m_total), i(256), i(k), ctypes.c_int(groups), ws, ctypes.c_size_t(ws_bytes), None)

    assert call(ctypes.c_void_p(0x10008), 1 << 24) == 2      # workspace not 16-byte aligned
    assert call(P, 1 << 24, m_total=200) == 3                 # MISALIGNED_LAYOUT, as without workspace
    assert call(P, 1 << 24, groups=0) == 1
    assert call(P, 1 << 24, k=500) == 2
    assert call(P, 1 << 24, m_total=0) == 0                   # empty problem: success, no launch


def test_masked_validation(lib):
    f = lib.dg_m_grouped_fp8_gemm_nt_masked
    i = ctypes.c_int64

    def call(groups=4, max_m=256, mm=P, k=512):
        return f(P, i(512), i(256 * 512), P, i(4), i(1), i(1024), P, i(512), i(256 * 512), P, i(4), i(1),
                 i(8), P, i(256), i(256 * 256), mm, ctypes.c_int(groups), i(max_m), i(256), i(k), i(128), None)

    assert call(groups=0) == 1
    assert call(groups=2000) == 2                        # beyond the device-side group limit
    assert call(mm=None) == 1
    assert call(k=100) == 2
    assert call(max_m=0) == 0


def test_cast_validation(lib):
    i = ctypes.c_int64
    f = lib.dg_per_token_cast_fp8
    assert f(P, i(512), P, i(512), P, i(4), i(1), i(8), i(500), 0, None) == 2   # k % 128
    assert f(P, i(256), P, i(512), P, i(4), i(1), i(8), i(512), 0, None) == 1   # ldx < k
    assert f(P, i(520), P, i(520), P, i(4), i(1), i(8), i(512), 0, None) == 2   # ldx*2 % 16 ok, ldq % 16 not
    assert f(None, i(512), P, i(512), P, i(4), i(1), i(8), i(512), 0, None) == 1
    assert f(P, i(512), P, i(512), P, i(4), i(1), i(0), i(512), 0, None) == 0
    g = lib.dg_per_block_cast_fp8
    assert g(P, i(512), P, i(512), P, i(4), i(1), i(8), i(100), 0, None) == 2


def test_packed_scale_entries_validation(lib):
    i = ctypes.c_int64
    f = lib.dg_fp8_gemm_nt_ue8m0

    def call(a=P, lda=512, sfa=P, b=P, sfb=P, d=P, m=128, n=256, k=512, ws=None, ws_bytes=0):
        return f(a, i(lda), sfa, i(1), i(128), b, i(512), sfb, i(1), i(2), d, i(256), i(m), i(n), i(k),
                 ws, ctypes.c_size_t(ws_bytes), None)

    assert call(sfa=None) == 1
    assert call(k=500) == 2
    assert call(m=0) == 0
    assert call(ws=ctypes.c_void_p(0x10004), ws_bytes=1 << 20) == 2       # misaligned workspace
    c = lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0
    assert c(P, i(512), P, i(1), i(256), P, i(512), i(1 << 20), P, i(2), i(1), i(4), P, i(256), P, i(200),
             i(256), i(512), 4, None) == 3                                # m_total % 128
    mk = lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0
    assert mk(P, i(512), i(1 << 20), P, i(1), i(256), i(1024), P, i(512), i(1 << 20), P, i(2), i(1), i(4),
              P, i(256), i(1 << 16), None, 4, i(256), i(256), i(512), i(128), None) == 1   # masked_m null
    pk = lib.dg_pack_ue8m0
    assert pk(None, i(4), i(1), P, i(1), i(1), i(8), i(4), None) == 1
    assert pk(P, i(4), i(1), ctypes.c_void_p(0x10002), i(1), i(1), i(8), i(4), None) == 2
    assert pk(P, i(-1), i(1), P, i(1), i(1), i(8), i(4), None) == 1
    assert pk(P, i(4), i(1), P, i(1), i(1), i(0), i(4), None) == 0


def test_accumulate_entry_validation(lib):
    i = ctypes.c_int64
    f = lib.dg_fp8_gemm_nt_acc

    def call(c=P, ldc=256, m=128, n=256):
        return f(P, i(512), P, i(4), i(1), P, i(512), P, i(4), i(1), c, i(ldc), P, i(256), i(m), i(n), i(512),
                 None, ctypes.c_size_t(0), None)

    assert call(c=None) == 1
    assert call(ldc=200) == 1                                  # ldc < n
    assert call(ldc=258) == 2                                  # ldc % 4
    assert call(c=ctypes.c_void_p(0x10008)) == 2               # c not 16-byte aligned
    assert call(c=None, m=0) == 0                              # empty problem


def test_grid_width_setting_and_the_pages_names():
    import moe_fp8_gemm_amd as dg
    try:
        dg.set_num_sms(7)
        assert dg.get_num_cus() == 7 and dg.get_num_sms() == 7
        dg.set_num_cus(0)                                    # back to every compute unit
        assert dg.get_num_sms() == dg.get_num_cus() > 7
    finally:
        dg.set_num_cus(0)


def test_forced_dense_plan_is_reported_and_checked():
    import moe_fp8_gemm_amd as dg
    try:
        dg.set_dense_plan(3, 5)                       # 128 x 64 tiles, 5 K splits
        assert dg.tile_config(100, 520, 1408) == (128, 64, 4)    # 11 blocks: 3 per split -> 4 splits
        assert dg.tile_config(100, 520, 1408, workspace=False) == (128, 64, 1)
        assert dg.workspace_size(100, 520, 1408) == 256 * 1024 + 1 * 9 * 4 * 128 * 64 * 4
        dg.set_dense_plan(4, 100)                     # more splits than K blocks: one block each
        assert dg.tile_config(64, 256, 640) == (64, 64, 5)
    finally:
        dg.set_dense_plan(-1)
    for inst, splits, status in [(7, 1, dg.DG_ERROR_INVALID_VALUE), (1, 0, dg.DG_ERROR_INVALID_VALUE),
                                 (5, 1, dg.DG_ERROR_NOT_SUPPORTED), (2, 2, dg.DG_ERROR_NOT_SUPPORTED),
                                 (6, 3, dg.DG_ERROR_NOT_SUPPORTED)]:
        with pytest.raises(dg.DgError) as e:
            dg.set_dense_plan(inst, splits)
        assert e.value.status == status
    dg.set_dense_plan(-1)


def test_contiguous_workspace_size_follows_the_plan():
    import moe_fp8_gemm_amd as dg
    hw = dg.get_num_cus()
    # G=8 over 66 blocks (the paired plan with 2 leftover blocks): one 128x128
    # fp32 partial tile per CU plus the 256 KiB counter block
    assert dg.contiguous_workspace_size(8448, 4096, 7168, 8) == 256 * 1024 + hw * 128 * 128 * 4
    try:
        dg.set_contiguous_plan(2)                      # one tile per block: never splits
        assert dg.contiguous_workspace_size(8448, 4096, 7168, 8) == 0
        dg.set_contiguous_plan(1)
        assert dg.contiguous_workspace_size(1024, 520, 256, 4) == 0     # 2 K blocks: too few to split
        full = dg.contiguous_workspace_size(1024, 520, 2048, 4)
        assert full > 0
        dg.set_num_cus(5)                               # the grid width does not change the plan
        assert dg.contiguous_workspace_size(1024, 520, 2048, 4) == full
    finally:
        dg.set_contiguous_plan(0)
        dg.set_num_cus(0)
    for bad in [(1000, 64, 256, 2), (1024, 64, 200, 2), (1024, 64, 256, 0), (0, 64, 256, 2)]:
        assert dg.contiguous_workspace_size(*bad) == 0


# ------------------------------------------------------------------ binding: scale shapes

def test_binding_rejects_scale_tensors_of_the_wrong_shape():
    """The kernels index scales from (rows, n, k) alone, so the binding checks
    the scale tensors' shapes per format before any pointer reaches the library."""
    import torch
    import moe_fp8_gemm_amd as m
    chk = m._check_scale_shapes
    f32 = lambda *s: torch.zeros(s, dtype=torch.float32)   # noqa: E731
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)     # noqa: E731
    # dense 300 x 264 x 1664: 13 K blocks -> 4 packed words; ceil(264/128) = 3 B blocks
    chk(f32(300, 13), f32(3, 13), (), 300, 264, 1664, False)
    chk(i32(300, 4), i32(3, 4), (), 300, 264, 1664, True)
    for sa, sb, packed in ((f32(300, 12), f32(3, 13), False),    # a missing K block
                           (f32(300, 13), f32(2, 13), False),    # floor(n/128) B blocks
                           (f32(299, 13), f32(3, 13), False),    # a missing row
                           (i32(300, 13), i32(3, 13), True),     # one int32 per K block, not packed words
                           (i32(300, 4), i32(3, 3), True)):
        with pytest.raises(ValueError):
            chk(sa, sb, (), 300, 264, 1664, packed)
    # grouped (masked): the group dimension leads both scale tensors
    chk(f32(5, 200, 5), f32(5, 3, 5), (5,), 200, 264, 640, False)
    with pytest.raises(ValueError):
        chk(f32(4, 200, 5), f32(5, 3, 5), (5,), 200, 264, 640, False)
    with pytest.raises(ValueError):
        chk(i32(5, 200, 5), i32(5, 3, 2), (5,), 200, 264, 640, True)


# ------------------------------------------------------------------ build: resource report

def test_build_resource_report_parser_and_no_scratch():
    """The build parses the compiler's kernel-resource-usage remarks; the last
    build's report (if present) shows no kernel with scratch memory or VGPR spills."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("dgfp8_build", os.path.join(ROOT, "moe_fp8_gemm_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    text = "\n".join([
        "x.hip:1:1: remark: Function Name: _Z1kv [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     TotalSGPRs: 104 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     VGPRs: 226 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 292 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     VGPRs Spill: 104 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     LDS Size [bytes/block]: 135168 [-Rpass-analysis=kernel-resource-usage]",
    ])
    k = b.parse_resource_remarks(text)
    assert k == [{"name": "_Z1kv", "sgpr": 104, "vgpr": 226, "agpr": 0, "scratch": 292, "vspill": 104, "lds": 135168}]
    report = os.path.join(ROOT, "moe_fp8_gemm_amd", "_build", "resource_usage.txt")
    if os.path.exists(report):
        rows = [l.split() for l in open(report).read().splitlines()[1:] if l.strip()]
        assert rows and all(r[3] == "0" and r[4] == "0" for r in rows), "a kernel uses scratch or spills VGPRs"


def test_absurd_sizes_and_strides_are_rejected_without_overflow(lib):
    # sizes whose products would overflow 64-bit arithmetic come back as
    # NOT_SUPPORTED (never a wrapped-around pass of the 32-bit offset check)
    big = 1 << 62
    assert _gemm(lib, m=big) == 2
    assert _gemm(lib, m=1 << 33) == 2
    assert _gemm(lib, ldd=big, n=256) == 2
    assert _gemm(lib, sfa_sm=big) == 2
    assert _gemm(lib, lda=big, k=512) == 2
    i = ctypes.c_int64
    size = lib.dg_fp8_gemm_nt_workspace_size
    size.restype = ctypes.c_size_t
    size.argtypes = [i, i, i]
    assert size(big, big, 128) == 0
    cfg = lib.dg_fp8_gemm_nt_tile_config
    bm, bn, sp = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    assert cfg(i(big), i(big), i(128), ctypes.c_size_t(0), ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(sp)) == 2
    f = lib.dg_per_token_cast_fp8
    assert f(P, i(big), P, i(512), P, i(4), i(1), i(8), i(512), 0, None) == 2     # ldx beyond 2^40
    assert f(P, i(512), P, i(512), P, i(4), i(1), i(big), i(512), 0, None) == 2   # rows beyond 2^40
    g = lib.dg_per_block_cast_fp8
    assert g(P, i(1 << 41), P, i(1 << 41), P, i(4), i(1), i(1 << 41), i(1 << 41), 0, None) == 2
    pack = lib.dg_pack_ue8m0
    assert pack(P, i(big), i(1), P, i(1), i(1), i(8), i(8), None) == 2
    m = lib.dg_m_grouped_fp8_gemm_nt_masked
    assert m(P, i(512), i(big), P, i(4), i(1), i(1024), P, i(512), i(256 * 512), P, i(4), i(1),
             i(8), P, i(256), i(256 * 256), P, ctypes.c_int(4), i(256), i(256), i(512), i(128), None) == 2
