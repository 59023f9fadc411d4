"""Helpers of the GPU parity tests: uploads, bf16 bit views, the acceptance check.

Acceptance for GEMM outputs, element-wise against the oracle's bf16 result o:
    |gpu - o| <= 8e-3 * |o| + 1e-3 * rms(o)      (rms over the compared elements)
and over the whole comparison  ||gpu - o||_F / ||o||_F <= 2e-3; NaN or Inf fails.
Quantizer codes and scales, routing and masking must match bit for bit.
"""
import numpy as np
import torch

TOL_REL = 8e-3
TOL_RMS = 1e-3
TOL_FRO = 2e-3
SENTINEL = 0x7FC1          # bf16 NaN bit pattern pre-filled into outputs


def device():
    return torch.device("cuda:0")


def upload_codes(q: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(q)).to(device()).view(torch.float8_e4m3fn)


def upload(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(device())


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor (any device)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def codes(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def sentinel_like(shape) -> torch.Tensor:
    return torch.full(shape, SENTINEL, dtype=torch.int16, device=device()).view(torch.bfloat16)


def assert_gemm_close(got_bits: np.ndarray, want_bits: np.ndarray, what: str = "") -> dict:
    g = bf16_to_f64(got_bits)
    o = bf16_to_f64(want_bits)
    assert g.shape == o.shape, what
    assert np.all(np.isfinite(g)), f"{what}: non-finite output at {np.argwhere(~np.isfinite(g))[:5].tolist()}"
    assert np.all(np.isfinite(o)), what
    rms = float(np.sqrt(np.mean(o * o))) if o.size else 0.0
    err = np.abs(g - o)
    bound = TOL_REL * np.abs(o) + TOL_RMS * rms
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:8]
        details = [(tuple(i), g[tuple(i)], o[tuple(i)]) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} elements out of tolerance, e.g. {details}")
    fro = float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-300))
    assert fro <= TOL_FRO, f"{what}: relative Frobenius error {fro}"
    return {"fro": fro, "max_ulp_like": float((err / np.maximum(np.abs(o), 1e-30)).max()) if o.size else 0.0}
