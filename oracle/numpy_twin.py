"""Pure-numpy transcription of the sequential selective scan, for tiny inputs only.

TEST INFRASTRUCTURE ONLY (see the package docstring).  It restates the same definition as
``ss_oracle.c`` independently -- vectorised over (batch, channel, state), one Python iteration per
time step -- so that a layout or marshalling slip in the C build shows up as a disagreement.

Definition followed (Mamba reading guide, "Método" and "O Mecanismo de Seleção (S6)"; IBM
explainer output equation and Mamba-block gate; aivaro.ru section 3 sketch for B_bar = delta*B,
the D*u skip and the zero initial state):
    dt = softplus(delta + delta_bias);  h = exp(dt*A) * h + dt * B * u;  y = C.h + D*u;
    out = y * silu(z).
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _as_f64(x):
    if x is None:
        return None
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return x.astype(np.float64)


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
             h0=None, zoh_exact=False):
    u, delta, B, C, z = (_as_f64(v) for v in (u, delta, B, C, z))
    A = np.asarray(A, dtype=np.float32).astype(np.float64)          # (d_inner, N)
    batch, L, d_inner = u.shape
    N = A.shape[1]
    s = delta + (0.0 if delta_bias is None else
                 np.asarray(delta_bias, np.float32).astype(np.float64)[None, None, :])
    dt = np.logaddexp(0.0, s) if delta_softplus else s              # softplus
    h = (np.zeros((batch, d_inner, N)) if h0 is None
         else np.array(h0, dtype=np.float64).reshape(batch, d_inner, N))
    out = np.empty((batch, L, d_inner))
    for t in range(L):
        dA = dt[:, t, :, None] * A[None, :, :]                      # (batch, d_inner, N)
        if zoh_exact:
            with np.errstate(divide="ignore", invalid="ignore"):
                fac = np.where(A[None] == 0.0, dt[:, t, :, None], np.expm1(dA) / A[None])
        else:
            fac = np.broadcast_to(dt[:, t, :, None], dA.shape)
        h = np.exp(dA) * h + fac * B[:, t, None, :] * u[:, t, :, None]
        y = np.einsum("bdn,bn->bd", h, C[:, t, :])
        if D is not None:
            y = y + np.asarray(D, np.float32).astype(np.float64)[None, :] * u[:, t, :]
        if z is not None:
            zt = z[:, t, :]
            y = y * (zt / (1.0 + np.exp(-zt)))
        out[:, t, :] = y
    return out, h
