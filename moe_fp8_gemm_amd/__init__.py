"""Python binding of libdgfp8: FP8 block-scaled GEMMs and FP8 casts for MI355X.

Argument marshalling only.  Each function checks dtypes/devices, hands raw
device pointers, strides and torch's current HIP stream to the C ABI declared
in ``include/dgfp8.h`` and raises ``DgError`` on a non-zero status.  All
arithmetic runs in the HIP kernels of ``libdgfp8.so``; there is no fallback:
importing this package fails loudly when the library has not been built.

Tensor conventions (torch): E4M3 operands are ``torch.float8_e4m3fn`` (or
``torch.uint8`` holding the codes), scales ``torch.float32`` with any
non-negative strides, outputs ``torch.bfloat16``.  Operands and scales are
passed as pairs ``(codes, scales)``.  The GEMMs also take packed UE8M0 scales
(``torch.int32`` words holding the exponents of 4 consecutive K blocks, see
``pack_ue8m0``): when both scale tensors are int32 the packed entry points run.
"""
from __future__ import annotations

import ctypes
import itertools
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdgfp8.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python moe_fp8_gemm_amd/build.py`")

lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int

_SIGNATURES = {
    "dg_status_string": ([_i32], ctypes.c_char_p),
    "dg_fp8_gemm_nt": ([_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _i64, _p, _i64,
                        _i64, _i64, _i64, _p], _i32),
    "dg_m_grouped_fp8_gemm_nt_contiguous": ([_p, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _i64,
                                             _p, _i64, _p, _i64, _i64, _i64, _i32, _p], _i32),
    "dg_m_grouped_fp8_gemm_nt_masked": ([_p, _i64, _i64, _p, _i64, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64,
                                         _i64, _p, _i64, _i64, _p, _i32, _i64, _i64, _i64, _i64, _p], _i32),
    "dg_per_token_cast_fp8": ([_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _i32, _p], _i32),
    "dg_per_token_cast_fp8_f32": ([_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _i32, _p], _i32),
    "dg_per_block_cast_fp8": ([_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _i32, _p], _i32),
    "dg_get_mk_alignment_for_contiguous_layout": ([], _i32),
    "dg_set_num_cus": ([_i32], _i32),
    "dg_get_num_cus": ([], _i32),
    "dg_fp8_gemm_nt_ws": ([_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _i64, _p, _i64,
                           _i64, _i64, _i64, _p, ctypes.c_size_t, _p], _i32),
    "dg_fp8_gemm_nt_workspace_size": ([_i64, _i64, _i64], ctypes.c_size_t),
    "dg_fp8_gemm_nt_tile_config": ([_i64, _i64, _i64, ctypes.c_size_t, _p, _p, _p], _i32),
    "dg_fp8_gemm_nt_ue8m0": ([_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _i64, _p, _i64,
                              _i64, _i64, _i64, _p, ctypes.c_size_t, _p], _i32),
    "dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0": ([_p, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64,
                                                   _i64, _p, _i64, _p, _i64, _i64, _i64, _i32, _p], _i32),
    "dg_m_grouped_fp8_gemm_nt_masked_ue8m0": ([_p, _i64, _i64, _p, _i64, _i64, _i64, _p, _i64, _i64, _p, _i64,
                                               _i64, _i64, _p, _i64, _i64, _p, _i32, _i64, _i64, _i64, _i64, _p],
                                              _i32),
    "dg_pack_ue8m0": ([_p, _i64, _i64, _p, _i64, _i64, _i64, _i64, _p], _i32),
    "dg_fp8_gemm_nt_acc": ([_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64,
                            _i64, _i64, _i64, _p, ctypes.c_size_t, _p], _i32),
    "dg_set_contiguous_plan": ([_i32], _i32),
    "dg_m_grouped_fp8_gemm_nt_contiguous_workspace_size": ([_i64, _i64, _i64, _i32], ctypes.c_size_t),
    "dg_m_grouped_fp8_gemm_nt_contiguous_ws": ([_p, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _i64,
                                                _p, _i64, _p, _i64, _i64, _i64, _i32, _p, ctypes.c_size_t, _p],
                                               _i32),
    "dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_ws": ([_p, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64,
                                                      _i64, _p, _i64, _p, _i64, _i64, _i64, _i32, _p,
                                                      ctypes.c_size_t, _p], _i32),
    "dg_set_dense_plan": ([_i32, _i32], _i32),
    "dg_fp8_gemm_nt_noalloc": ([_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _i64, _p, _i64,
                                _i64, _i64, _i64, _p], _i32),
}
for _name, (_args, _res) in _SIGNATURES.items():
    _f = getattr(lib, _name)
    _f.argtypes = _args
    _f.restype = _res

DG_SUCCESS = 0
DG_ERROR_INVALID_VALUE = 1
DG_ERROR_NOT_SUPPORTED = 2
DG_ERROR_MISALIGNED_LAYOUT = 3
DG_ERROR_LAUNCH = 4
DG_ERROR_SCRATCH_LIMIT = 5


class DgError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib.dg_status_string(status).decode()}")


def _check(status: int, where: str) -> None:
    if status != DG_SUCCESS:
        raise DgError(status, where)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _codes(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise TypeError(f"{name} must be float8_e4m3fn or uint8 codes, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.stride(-1) != 1:
        raise ValueError(f"{name} must be K-major (unit stride along K)")
    return t


def _scales(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype not in (torch.float32, torch.int32) or not t.is_cuda:
        raise TypeError(f"{name} must be a float32 (or packed UE8M0 int32) device tensor")
    return t


def _packed(sa: torch.Tensor, sb: torch.Tensor) -> bool:
    """True for packed UE8M0 scales (both int32), False for fp32 (both float32)."""
    if sa.dtype != sb.dtype:
        raise TypeError("sfa and sfb must both be float32 or both be packed int32")
    return sa.dtype == torch.int32


def _scale_words(k: int, packed: bool) -> int:
    """Scale entries per row along K: one per 128-wide K block (fp32), or one
    int32 word per 4 K blocks (packed UE8M0)."""
    kb = k // 128
    return (kb + 3) // 4 if packed else kb


def _check_scale_shapes(sa: torch.Tensor, sb: torch.Tensor, lead: tuple, rows_a: int, n: int, k: int,
                        packed: bool) -> None:
    """The kernels index the scale arrays from (rows, n, k) alone, so a scale
    tensor of the wrong shape would be read out of bounds: reject it here.
    lead: leading (group) dimensions of both scale tensors."""
    if k % 128:
        return                       # the library rejects K % 128 != 0 itself
    kw = _scale_words(k, packed)
    want_a = tuple(lead) + (rows_a, kw)
    want_b = tuple(lead) + ((n + 127) // 128, kw)
    what = "packed UE8M0 int32" if packed else "float32"
    if tuple(sa.shape) != want_a:
        raise ValueError(f"sfa ({what}) must have shape {want_a}, got {tuple(sa.shape)}")
    if tuple(sb.shape) != want_b:
        raise ValueError(f"sfb ({what}) must have shape {want_b}, got {tuple(sb.shape)}")


def _out_bf16(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.bfloat16 or not t.is_cuda or t.stride(-1) != 1:
        raise TypeError(f"{name} must be a bfloat16 device tensor with unit column stride")
    return t


_AUTO = "auto"
_workspaces = {}      # (device index, stream handle) -> zero-initialised workspace


def workspace_size(m: int, n: int, k: int) -> int:
    """Bytes of split-K workspace fp8_gemm_nt can use for this problem (0: never splits)."""
    return int(lib.dg_fp8_gemm_nt_workspace_size(int(m), int(n), int(k)))


def tile_config(m: int, n: int, k: int, workspace: bool = True) -> Tuple[int, int, int]:
    """(block_m, block_n, splits) fp8_gemm_nt uses for this problem (with the auto workspace, or none)."""
    bm, bn, sp = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    ws = workspace_size(m, n, k) if workspace else 0
    _check(lib.dg_fp8_gemm_nt_tile_config(int(m), int(n), int(k), ws, ctypes.byref(bm), ctypes.byref(bn),
                                          ctypes.byref(sp)), "dg_fp8_gemm_nt_tile_config")
    return bm.value, bn.value, sp.value


def _auto_workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    # One zero-filled workspace per (device, stream), grown on demand.  Calls
    # leave its counter block zero, so every later call on that stream reuses
    # it; calls on different streams, which may overlap, never share one.  It is
    # allocated (and zero-filled) on the stream that uses it, so the caching
    # allocator hands its memory to no other stream while that one may use it.
    idx = device.index if device.index is not None else torch.cuda.current_device()
    key = (idx, torch.cuda.current_stream(idx).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _workspace_arg(workspace, device: torch.device, need: int) -> Tuple[int, int]:
    """(pointer, bytes) of the split-K workspace argument: "auto" -> the cached
    per-(device, stream) buffer when the problem can use one, None -> none."""
    if isinstance(workspace, str):
        if workspace != _AUTO:
            raise ValueError("workspace must be 'auto', None or a tensor")
        workspace = _auto_workspace(device, need) if need > 0 else None
    if workspace is None:
        return 0, 0
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous device tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def fp8_gemm_nt(a: Tuple[torch.Tensor, torch.Tensor], b: Tuple[torch.Tensor, torch.Tensor],
                d: torch.Tensor, c: Optional[torch.Tensor] = None, workspace=_AUTO) -> torch.Tensor:
    """d[m, n] = bf16( A . B^T [+ c] ) with per-(row, 128-K) A scales and per-128x128 B scales.

    a = (codes [m, k], sfa [m, k/128]); b = (codes [n, k], sfb [ceil(n/128), k/128]);
    d bf16 [m, n] is overwritten and returned; c, when given, is an fp32 [m, n]
    addend (fp32 scales only).  Packed UE8M0 scales (both int32) are
    [m, ceil(k/512)] and [ceil(n/128), ceil(k/512)].  ``workspace``: "auto" (a
    cached buffer per device and stream, enabling split-K for small m), None
    (never split), or a zero-initialised uint8 device tensor of at least
    ``workspace_size(m, n, k)`` bytes (calls that may overlap need distinct ones).
    """
    (qa, sa), (qb, sb) = a, b
    _codes(qa, "a"); _codes(qb, "b"); _scales(sa, "sfa"); _scales(sb, "sfb"); _out_bf16(d, "d")
    if qa.dim() != 2 or qb.dim() != 2 or d.dim() != 2:
        raise ValueError("a, b and d must be 2-D")
    m, k = qa.shape
    n = qb.shape[0]
    if qb.shape[1] != k or d.shape != (m, n):
        raise ValueError("shape mismatch")
    _check_scale_shapes(sa, sb, (), m, n, k, _packed(sa, sb))
    ws_ptr, ws_bytes = _workspace_arg(workspace, d.device, workspace_size(m, n, k))
    packed = _packed(sa, sb)
    if c is not None:
        if packed:
            raise NotImplementedError("the accumulating GEMM takes fp32 scales")
        if c.dtype != torch.float32 or not c.is_cuda or c.shape != (m, n) or c.stride(1) != 1:
            raise TypeError("c must be a float32 device tensor [m, n] with unit column stride")
        _check(lib.dg_fp8_gemm_nt_acc(qa.data_ptr(), qa.stride(0), sa.data_ptr(), sa.stride(0), sa.stride(1),
                                      qb.data_ptr(), qb.stride(0), sb.data_ptr(), sb.stride(0), sb.stride(1),
                                      c.data_ptr(), c.stride(0), d.data_ptr(), d.stride(0), m, n, k,
                                      ws_ptr or None, ws_bytes, _stream()), "dg_fp8_gemm_nt_acc")
        return d
    fn = lib.dg_fp8_gemm_nt_ue8m0 if packed else lib.dg_fp8_gemm_nt_ws
    _check(fn(qa.data_ptr(), qa.stride(0), sa.data_ptr(), sa.stride(0), sa.stride(1),
              qb.data_ptr(), qb.stride(0), sb.data_ptr(), sb.stride(0), sb.stride(1),
              d.data_ptr(), d.stride(0), m, n, k, ws_ptr or None, ws_bytes, _stream()),
           "dg_fp8_gemm_nt")
    return d


def fp8_gemm_nt_noalloc(a: Tuple[torch.Tensor, torch.Tensor], b: Tuple[torch.Tensor, torch.Tensor],
                        d: torch.Tensor) -> torch.Tensor:
    """fp8_gemm_nt (fp32 scales) for callers that cannot allocate: split-K runs in
    the library's static per-device scratch instead of a workspace.  Raises
    DgError (DG_ERROR_SCRATCH_LIMIT) when the problem's split plan needs more
    scratch than that holds.  Calls that may overlap on one device race."""
    (qa, sa), (qb, sb) = a, b
    _codes(qa, "a"); _codes(qb, "b"); _scales(sa, "sfa"); _scales(sb, "sfb"); _out_bf16(d, "d")
    if qa.dim() != 2 or qb.dim() != 2 or d.dim() != 2:
        raise ValueError("a, b and d must be 2-D")
    m, k = qa.shape
    n = qb.shape[0]
    if qb.shape[1] != k or d.shape != (m, n):
        raise ValueError("shape mismatch")
    if _packed(sa, sb):
        raise NotImplementedError("the no-allocation GEMM takes fp32 scales")
    _check_scale_shapes(sa, sb, (), m, n, k, False)
    _check(lib.dg_fp8_gemm_nt_noalloc(qa.data_ptr(), qa.stride(0), sa.data_ptr(), sa.stride(0), sa.stride(1),
                                      qb.data_ptr(), qb.stride(0), sb.data_ptr(), sb.stride(0), sb.stride(1),
                                      d.data_ptr(), d.stride(0), m, n, k, _stream()), "dg_fp8_gemm_nt_noalloc")
    return d


def contiguous_workspace_size(m_total: int, n: int, k: int, num_groups: int) -> int:
    """Bytes of split-K workspace m_grouped_fp8_gemm_nt_contiguous can use (0: never splits)."""
    return int(lib.dg_m_grouped_fp8_gemm_nt_contiguous_workspace_size(int(m_total), int(n), int(k),
                                                                       int(num_groups)))


def m_grouped_fp8_gemm_nt_contiguous(a, b, d: torch.Tensor, m_indices: torch.Tensor,
                                     workspace=_AUTO) -> torch.Tensor:
    """Contiguous MoE layout: a = (codes [m_total, k], sfa [m_total, k/128]),
    b = (codes [G, n, k], sfb [G, ceil(n/128), k/128]), d bf16 [m_total, n],
    m_indices int32 [m_total] (-1 on padding rows, which are left untouched).
    ``workspace`` as for fp8_gemm_nt ("auto", None, or a zero-initialised uint8
    device tensor of at least ``contiguous_workspace_size(...)`` bytes): with
    one, the blocks that the paired plan leaves to its second launch split K."""
    (qa, sa), (qb, sb) = a, b
    _codes(qa, "a"); _codes(qb, "b"); _scales(sa, "sfa"); _scales(sb, "sfb"); _out_bf16(d, "d")
    if m_indices.dtype != torch.int32 or not m_indices.is_cuda:
        raise TypeError("m_indices must be an int32 device tensor")
    if qa.dim() != 2 or qb.dim() != 3 or d.dim() != 2:
        raise ValueError("a must be [m_total, k], b [G, n, k] and d [m_total, n]")
    m_total, k = qa.shape
    g, n, _ = qb.shape
    if qb.shape[2] != k or d.shape != (m_total, n) or m_indices.shape != (m_total,) or m_indices.stride(0) != 1:
        raise ValueError("shape mismatch")
    if sa.dim() != 2 or sb.dim() != 3:
        raise ValueError("sfa must be [m_total, k-words] and sfb [G, ceil(n/128), k-words]")
    _check_scale_shapes(sa, sb[0], (), m_total, n, k, _packed(sa, sb))
    if sb.shape[0] != g:
        raise ValueError(f"sfb has {sb.shape[0]} groups, b has {g}")
    ws_ptr, ws_bytes = _workspace_arg(workspace, d.device, contiguous_workspace_size(m_total, n, k, g))
    fn = (lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_ws if _packed(sa, sb)
          else lib.dg_m_grouped_fp8_gemm_nt_contiguous_ws)
    _check(fn(
        qa.data_ptr(), qa.stride(0), sa.data_ptr(), sa.stride(0), sa.stride(1),
        qb.data_ptr(), qb.stride(1), qb.stride(0),
        sb.data_ptr(), sb.stride(1), sb.stride(2), sb.stride(0),
        d.data_ptr(), d.stride(0), m_indices.data_ptr(), m_total, n, k, g, ws_ptr or None, ws_bytes, _stream()),
        "dg_m_grouped_fp8_gemm_nt_contiguous")
    return d


def m_grouped_fp8_gemm_nt_masked(a, b, d: torch.Tensor, masked_m: torch.Tensor,
                                 expected_m: int) -> torch.Tensor:
    """Masked MoE layout: a = (codes [G, max_m, k], sfa [G, max_m, k/128]),
    b = (codes [G, n, k], sfb [G, ceil(n/128), k/128]), d bf16 [G, max_m, n],
    masked_m int32 [G] read on the device; rows >= masked_m[g] are left untouched."""
    (qa, sa), (qb, sb) = a, b
    _codes(qa, "a"); _codes(qb, "b"); _scales(sa, "sfa"); _scales(sb, "sfb"); _out_bf16(d, "d")
    if masked_m.dtype != torch.int32 or not masked_m.is_cuda:
        raise TypeError("masked_m must be an int32 device tensor")
    if qa.dim() != 3 or qb.dim() != 3 or d.dim() != 3:
        raise ValueError("a must be [G, max_m, k], b [G, n, k] and d [G, max_m, n]")
    g, max_m, k = qa.shape
    n = qb.shape[1]
    if qb.shape != (g, n, k) or d.shape != (g, max_m, n) or masked_m.shape != (g,) or masked_m.stride(0) != 1:
        raise ValueError("shape mismatch")
    _check_scale_shapes(sa, sb, (g,), max_m, n, k, _packed(sa, sb))
    fn = lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0 if _packed(sa, sb) else lib.dg_m_grouped_fp8_gemm_nt_masked
    _check(fn(
        qa.data_ptr(), qa.stride(1), qa.stride(0),
        sa.data_ptr(), sa.stride(1), sa.stride(2), sa.stride(0),
        qb.data_ptr(), qb.stride(1), qb.stride(0),
        sb.data_ptr(), sb.stride(1), sb.stride(2), sb.stride(0),
        d.data_ptr(), d.stride(1), d.stride(0),
        masked_m.data_ptr(), g, max_m, n, k, int(expected_m), _stream()),
        "dg_m_grouped_fp8_gemm_nt_masked")
    return d


def _cast_out(rows: int, k: int, device, q: Optional[torch.Tensor], sf: Optional[torch.Tensor], sf_rows: int):
    if q is None:
        q = torch.empty((rows, k), dtype=torch.float8_e4m3fn, device=device)
    if sf is None:
        sf = torch.empty((sf_rows, k // 128), dtype=torch.float32, device=device)
    if tuple(q.shape) != (rows, k) or q.dtype not in (torch.float8_e4m3fn, torch.uint8) or not q.is_cuda:
        raise ValueError("q must be an E4M3 (or uint8) device tensor of shape (%d, %d)" % (rows, k))
    if tuple(sf.shape) != (sf_rows, k // 128) or sf.dtype != torch.float32 or not sf.is_cuda:
        raise ValueError("sf must be an fp32 device tensor of shape (%d, %d)" % (sf_rows, k // 128))
    return q, sf


def per_token_cast_fp8(x: torch.Tensor, ue8m0: bool = False, q: Optional[torch.Tensor] = None,
                       sf: Optional[torch.Tensor] = None):
    """x bf16 or fp32 [m, k] -> (E4M3 codes [m, k], fp32 scales [m, k/128]), 1x128 blocks."""
    if x.dtype not in (torch.bfloat16, torch.float32) or not x.is_cuda or x.stride(-1) != 1:
        raise TypeError("x must be a bf16 or fp32 device tensor with unit column stride")
    m, k = x.shape
    q, sf = _cast_out(m, k, x.device, q, sf, m)
    fn = lib.dg_per_token_cast_fp8_f32 if x.dtype == torch.float32 else lib.dg_per_token_cast_fp8
    _check(fn(x.data_ptr(), x.stride(0), q.data_ptr(), q.stride(0), sf.data_ptr(), sf.stride(0), sf.stride(1),
              m, k, int(bool(ue8m0)), _stream()), "per_token_cast_fp8")
    return q, sf


def per_block_cast_fp8(w: torch.Tensor, ue8m0: bool = False, q: Optional[torch.Tensor] = None,
                       sf: Optional[torch.Tensor] = None):
    """w fp32 [n, k] -> (E4M3 codes [n, k], fp32 scales [ceil(n/128), k/128]), 128x128 blocks."""
    if w.dtype != torch.float32 or not w.is_cuda or w.stride(-1) != 1:
        raise TypeError("w must be an fp32 device tensor with unit column stride")
    n, k = w.shape
    q, sf = _cast_out(n, k, w.device, q, sf, (n + 127) // 128)
    _check(lib.dg_per_block_cast_fp8(w.data_ptr(), w.stride(0), q.data_ptr(), q.stride(0), sf.data_ptr(),
                                     sf.stride(0), sf.stride(1), n, k, int(bool(ue8m0)), _stream()),
           "per_block_cast_fp8")
    return q, sf


def pack_ue8m0(sf: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 scales [..., rows, kblocks] -> packed UE8M0 int32 words [..., rows, ceil(kblocks/4)].

    Byte j of word w is the biased exponent of scale 4w+j rounded up to a power of
    two (exact for the power-of-two scales the casts produce with ``ue8m0=True``).
    Leading dimensions (e.g. groups) are handled one matrix at a time; any strides.
    """
    if sf.dtype != torch.float32 or not sf.is_cuda or sf.dim() < 2:
        raise TypeError("sf must be a float32 device tensor of at least 2 dims")
    rows, kb = sf.shape[-2], sf.shape[-1]
    words = (kb + 3) // 4
    if out is None:
        out = torch.empty(sf.shape[:-1] + (words,), dtype=torch.int32, device=sf.device)
    if out.dtype != torch.int32 or tuple(out.shape) != tuple(sf.shape[:-1]) + (words,) or not out.is_cuda:
        raise ValueError("out must be an int32 device tensor of shape [..., rows, ceil(kblocks/4)]")
    for idx in itertools.product(*(range(x) for x in sf.shape[:-2])):
        s, o = sf[idx], out[idx]
        _check(lib.dg_pack_ue8m0(s.data_ptr(), s.stride(0), s.stride(1), o.data_ptr(), o.stride(0), o.stride(1),
                                 rows, kb, _stream()), "dg_pack_ue8m0")
    return out


def get_mk_alignment_for_contiguous_layout() -> int:
    return lib.dg_get_mk_alignment_for_contiguous_layout()


def set_num_cus(num_cus: int) -> None:
    _check(lib.dg_set_num_cus(int(num_cus)), "dg_set_num_cus")


def get_num_cus() -> int:
    return lib.dg_get_num_cus()


def set_contiguous_plan(plan: int) -> None:
    """Contiguous grouped GEMM plan: 0 cost model (default), 1 paired 256-row
    tiles + leftover 128-row blocks, 2 one tile per 128-row block.  Same bits."""
    _check(lib.dg_set_contiguous_plan(int(plan)), "dg_set_contiguous_plan")


def set_dense_plan(instance: int, splits: int = 1) -> None:
    """Force the dense GEMM's kernel instance and K splits (instance < 0: cost
    model, the default).  Instance numbers as in dg_set_dense_plan."""
    _check(lib.dg_set_dense_plan(int(instance), int(splits)), "dg_set_dense_plan")


# The pages' names for the persistent-grid width (page ssnai.com DeepGEMM
# analysis, 配置与调优建议: run-time tuning with set_num_sms).  On MI355X the unit
# is the compute unit; the tensor-core-utilisation and programmatic-launch knobs
# named beside it have no counterpart here.
set_num_sms = set_num_cus
get_num_sms = get_num_cus

