"""Tolerance rules and conversions shared by the GPU parity tests."""

import numpy as np
import torch

# Max |GPU - oracle| allowed per element, by storage dtype.
TOL = {"f16": 2e-3, "bf16": 1e-2}


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a fp16/bf16 tensor to a float64 array (on the CPU)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float64).tiny)
    return 0.5 * np.exp2(np.floor(np.log2(ax)) - 7)


def allowed(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Per-element bound.  bf16 outputs with |oracle| >= 2 may also be off by the final
    rounding to bf16 itself (half an ulp is 7.8e-3 in [2, 4) and 1.6e-2 in [4, 8)), so
    there the bound is the gate plus half an ulp of the oracle value."""
    tol = np.full(ref.shape, TOL[dtype])
    if dtype == "bf16":
        big = np.abs(ref) >= 2
        tol = np.where(big, TOL[dtype] + bf16_half_ulp(ref), tol)
    return tol


def check(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = allowed(ref, dtype)
    bad = err > bound
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {err.size} elements over the bound; max err {err.max():.3e}; "
            f"first at {idx.tolist()} got {got[tuple(idx[0])]:.6f} ref {ref[tuple(idx[0])]:.6f}"
        )
    return float(err.max())
