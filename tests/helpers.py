"""Shared helpers for the GPU parity tests: device upload of generator arrays and the
elementwise tolerance check |gpu - ref| <= atol + rtol * |ref|."""
from __future__ import annotations

import numpy as np
import torch

# Tolerances stated for the selective scan: float32 inputs 1e-4, bfloat16 inputs 2e-2 (rel and
# abs, elementwise), float32 state.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def dev(x, device="cuda"):
    """numpy float32 or uint16 (bf16 bits) -> torch tensor on the GPU with the same bytes."""
    if x is None:
        return None
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(device)
    if x.dtype == np.float32:
        return torch.from_numpy(x).to(device)
    raise TypeError(x.dtype)


def host(t: torch.Tensor) -> np.ndarray:
    """GPU tensor -> float64 numpy (bf16 widened exactly)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_close(got, want, tol, what, frac_report=None):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    err = np.abs(got - want)
    bound = tol + tol * np.abs(want)
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements outside atol=rtol={tol}; worst at "
            f"{tuple(int(v) for v in i)}: got {got[i]!r} want {want[i]!r}")
    rel = err / (np.abs(want) + 1e-30)
    return float(err.max(initial=0.0)), float(np.median(rel)) if rel.size else 0.0
