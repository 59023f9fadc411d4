"""Every pair of E4M3 codes through the GEMM, bit for bit against the oracle.

The product of two E4M3 values has at most 8 significant bits, so it is
exact in fp32 and in bf16.  Row i of A holds code i at all 128 positions of
one K block and row j of B holds code j; with A scales 2^-7 and B scales 1,

    D[i, j] = 2^-7 * sum_{k < 128} dec(i) * dec(j) = dec(i) * dec(j)

exactly, whatever the summation order.  A code decoded differently by the
matrix cores, on either MFMA port (B rows feed one, A rows the other) and at
any K position, therefore changes bits of D.  This pins the hardware's E4M3
decode (OCP E4M3 "FN": bias 7, subnormals, max 448; pages on DeepGEMM: FP8
E4M3 operands, page "企业官网建设流程全解析" section 2.3) against the oracle's
table.  The two NaN codes (0x7F, 0xFF) are outside the contract: their rows
hold code 0.  The sign of an exact zero sum is not fixed by the definition
(it depends on the order of the additions and on the initial zero), so zero
results are compared as values.
"""
import numpy as np
import pytest
import torch

from oracle import e4m3
from oracle import gemm as ogemm
from gpu_util import bits, upload, upload_codes

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import moe_fp8_gemm_amd as dg  # noqa: E402

NAN_CODES = (0x7F, 0xFF)


def _operands():
    codes = np.arange(256, dtype=np.uint8)
    codes[list(NAN_CODES)] = 0
    q = np.repeat(codes[:, None], 128, axis=1)                 # [256, 128]: row c holds code c
    sa = np.full((256, 1), 2.0 ** -7, dtype=np.float32)
    sb = np.ones((2, 1), dtype=np.float32)
    return codes, q, sa, sb


def _check(got_bits, codes, q, sa, sb):
    want = ogemm.gemm_nt(q, sa, q, sb)
    # the construction: the oracle's result is the plain product of the decoded codes
    dec = e4m3.decode(codes)
    assert np.array_equal(ogemm.as_float(want), np.outer(dec, dec))
    got, exp = ogemm.as_float(got_bits), ogemm.as_float(want)
    valid = np.ones(256, dtype=bool)
    valid[list(NAN_CODES)] = False
    mask = np.outer(valid, valid)
    nonzero = mask & (exp != 0)
    bad = np.argwhere(nonzero & (got_bits != want))
    assert bad.size == 0, f"{len(bad)} code pairs differ, first (a, b) = {bad[:5].tolist()}"
    assert np.array_equal(got[mask & (exp == 0)], exp[mask & (exp == 0)])


@pytest.mark.parametrize("packed", [False, True])
def test_every_e4m3_code_pair(packed):
    codes, q, sa, sb = _operands()
    qt = upload_codes(q)
    sa_t, sb_t = upload(sa), upload(sb)
    if packed:
        sa_t, sb_t = dg.pack_ue8m0(sa_t), dg.pack_ue8m0(sb_t)
    d = torch.empty((256, 256), dtype=torch.bfloat16, device=qt.device)
    dg.fp8_gemm_nt((qt, sa_t), (qt, sb_t), d)
    torch.cuda.synchronize()
    _check(bits(d), codes, q, sa, sb)


@pytest.mark.parametrize("inst", [0, 1, 2, 3, 4, 6])
def test_every_e4m3_code_pair_on_every_instance(inst):
    """The same on each dense tile instance (each has its own fragment layout)."""
    codes, q, sa, sb = _operands()
    qt = upload_codes(q)
    d = torch.empty((256, 256), dtype=torch.bfloat16, device=qt.device)
    dg.set_dense_plan(inst, 1)
    try:
        dg.fp8_gemm_nt((qt, upload(sa)), (qt, upload(sb)), d)
        torch.cuda.synchronize()
    finally:
        dg.set_dense_plan(-1, 1)
    _check(bits(d), codes, q, sa, sb)
