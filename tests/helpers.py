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


class Errors:
    """Elementwise check |got - want| <= tol + tol*|want| over blocks, keeping the worst errors."""

    def __init__(self, what, tol):
        self.what, self.tol = what, tol
        self.max_abs = 0.0
        self.max_rel = 0.0      # |got - want| / |want| over elements with |want| >= 1e-3
        self.worst = 0.0        # max of err / bound (<= 1 passes)
        self.n = 0

    def add(self, got, want, where=""):
        got = np.asarray(got, dtype=np.float64)
        want = np.asarray(want, dtype=np.float64)
        assert got.shape == want.shape, (self.what, got.shape, want.shape)
        err = np.subtract(got, want)
        np.abs(err, out=err)
        bound = np.abs(want)
        big = bound >= 1e-3
        if big.any():
            self.max_rel = max(self.max_rel, float((err[big] / bound[big]).max()))
        bound *= self.tol
        bound += self.tol
        ratio = err / bound
        self.n += err.size
        if err.size:
            self.max_abs = max(self.max_abs, float(err.max()))
            w = float(ratio.max())            # NaN propagates and fails the check below
            self.worst = max(self.worst, w) if w == w else float("nan")
            if not w <= 1.0:
                bad = ~(ratio <= 1.0)
                i = np.unravel_index(np.argmax(np.where(bad, np.inf, ratio)), err.shape)
                raise AssertionError(
                    f"{self.what}{where}: {int(bad.sum())} of {bad.size} elements outside "
                    f"atol=rtol={self.tol}; worst at {tuple(int(v) for v in i)}: got "
                    f"{got[i]!r} want {want[i]!r}")

    def report(self):
        print(f"  {self.what}: {self.n} elements, max abs err {self.max_abs:.3e}, max rel err "
              f"{self.max_rel:.3e} (|ref| >= 1e-3), worst err/bound {self.worst:.3f} at "
              f"tol {self.tol}", flush=True)


def check_every_row(out, h_last, reference, what, *, out_tol, h_tol, block=1024):
    """Compare a (batch, L, d_inner) GPU output and its (batch, d_inner, N) final state with a
    reference evaluated block by block: reference(b, d0, d1) returns the fp64 (d1 - d0, L)
    outputs and (d1 - d0, N) final states of rows (b, d0..d1-1).  Every row is compared; the
    achieved errors are printed."""
    batch, _, d_inner = out.shape
    e_out, e_h = Errors(f"{what} out", out_tol), Errors(f"{what} h_last", h_tol)
    for b in range(batch):
        for d0 in range(0, d_inner, block):
            d1 = min(d_inner, d0 + block)
            r, rh = reference(b, d0, d1)
            got = out[b, :, d0:d1].float().t().contiguous().cpu().numpy()
            e_out.add(got, r, f" (b={b}, d={d0}..{d1 - 1})")
            del got, r
            if h_last is not None:
                e_h.add(h_last[b, d0:d1].cpu().numpy(), rh, f" (b={b}, d={d0}..{d1 - 1})")
    e_out.report()
    if h_last is not None:
        e_h.report()
