"""Comparison rules shared by the GPU parity tests.

Tolerances (stated for the attention forward in this project's goals):
  * O:   max |O_gpu - O_oracle| <= 1e-2.  For a bfloat16 O the output's own
         rounding is not counted against the kernel: the bound becomes
         1e-2 + half a bf16 ulp of |O_oracle| (bf16 keeps 8 significant bits,
         so an exactly computed value of magnitude in [4, 8) may still land
         0.0156 away once stored).  A float32 O gets the plain 1e-2.
  * LSE: max |LSE_gpu - LSE_oracle| <= 1e-3, and rows whose oracle LSE is
         -inf (no allowed key) must be exactly -inf with O exactly 0.
  * no NaN anywhere.
"""
from __future__ import annotations

import numpy as np
import torch

O_TOL = 1e-2
LSE_TOL = 1e-3


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8.0), 0.0)


def check(o_gpu, lse_gpu, o_ref, lse_ref, out_dtype: str, label: str = ""):
    """o_gpu / lse_gpu: numpy float64 of the GPU result (same shapes as the refs)."""
    assert not np.isnan(o_gpu).any(), f"{label}: NaN in O"
    tol = O_TOL + (bf16_half_ulp(o_ref) if out_dtype == "bf16" else 0.0)
    err = np.abs(o_gpu - o_ref)
    bad = err > tol
    if bad.any():
        idx = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(
            f"{label}: O mismatch at {idx}: gpu={o_gpu[idx]!r} oracle={o_ref[idx]!r} "
            f"err={err[idx]:.3e} tol={np.broadcast_to(tol, err.shape)[idx]:.3e} "
            f"({bad.sum()} of {bad.size} outside)")
    if lse_gpu is None:
        return float(err.max()) if err.size else 0.0, 0.0
    assert not np.isnan(lse_gpu).any(), f"{label}: NaN in LSE"
    ninf = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), ninf), f"{label}: -inf LSE rows differ"
    lerr = np.abs(lse_gpu[~ninf] - lse_ref[~ninf]) if (~ninf).any() else np.zeros(1)
    assert np.isfinite(lerr).all(), f"{label}: non-finite LSE"
    assert lerr.max() <= LSE_TOL, f"{label}: LSE error {lerr.max():.3e} > {LSE_TOL}"
    return float(err.max()) if err.size else 0.0, float(lerr.max())


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
