"""Thin ctypes binding of libssscan.so (include/ss_scan.h) for torch tensors.

Argument marshalling only: every step of the scan runs in the library's HIP kernels.  torch
provides device memory and the stream.  There is no fallback: if the library is missing or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssscan.so")

SS_OK, SS_ERR_INVALID_ARG, SS_ERR_UNSUPPORTED, SS_ERR_HIP = 0, 1, 2, 3
SS_F32, SS_BF16 = 0, 1
SS_FLAG_ZOH_EXACT = 1
SS_FLAG_STATES_GIVEN = 2

# Every symbol declared in include/ss_scan.h, with its ctypes signature.
_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_u32 = ctypes.c_uint32
SIGNATURES = {
    "ss_scan_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
                           _i64, _i64, _i64, _i64, _i32, _vp, _sz, _vp]),
    "ss_scan_fwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i32]),
    "ss_scan_fwd_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp,
                                   _vp, _vp, _i64, _i64, _i64, _i64, _i32, _vp]),
    "ss_scan_fwd_ex": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp,
                              _vp, _i64, _i64, _i64, _i64, _i32, _vp, _sz, _i32, _u32, _vp]),
    "ss_scan_fwd_ex_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i32, _i32]),
    "ss_scan_fwd_states": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp,
                                  _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i32, _vp, _sz, _vp]),
    "ss_scan_fwd_states_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "ss_scan_fwd_conv": (_i32, [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                ctypes.c_int, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i32, _vp,
                                _sz, _i32, _u32, _vp]),
    "ss_scan_bwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
                           _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                           _i32, _vp, _sz, _u32, _vp]),
    "ss_scan_bwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i32]),
    "ss_scan2_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp,
                            _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i32, _vp]),
    "ss_state_update_conv": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _vp, ctypes.c_int, _vp, _i64, _i64, _i64, _i32, _u32,
                                    _vp]),
    "ss_state_update": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp,
                               _i64, _i64, _i64, _i32, _vp]),
    "ss_state_update_ex": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int,
                                  _vp, _i64, _i64, _i64, _i32, _u32, _vp]),
    "ss_status_string": (ctypes.c_char_p, [_i32]),
    "ss_last_error": (ctypes.c_char_p, []),
    "ss_version": (ctypes.c_int, []),
}

_lib = None


class SSError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library, with argument types set.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m selective_state_space_36_amd.build`"
                " (or __graft_entry__.build())")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _check(status: int) -> None:
    if status != SS_OK:
        msg = lib().ss_last_error().decode() or lib().ss_status_string(status).decode()
        raise SSError(status, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SS_F32
    if t.dtype == torch.bfloat16:
        return SS_BF16
    raise TypeError(f"io tensors must be float32 or bfloat16, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, shape=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def workspace_bytes(batch, seqlen, d_inner, d_state, dtype=torch.bfloat16, nseg=None) -> int:
    code = SS_BF16 if dtype == torch.bfloat16 else SS_F32
    if nseg is None:
        return int(lib().ss_scan_fwd_workspace_bytes(batch, seqlen, d_inner, d_state, code))
    return int(lib().ss_scan_fwd_ex_workspace_bytes(batch, seqlen, d_inner, d_state, code, nseg))


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True, h0=None,
             return_last_state=False, out=None, h_last=None, workspace=None, nseg=None,
             zoh_exact=False, stream=None):
    """Prefill selective scan on the GPU (ss_scan_fwd / ss_scan_fwd_ex).

    u, delta, z: (batch, L, d_inner); B, C: (batch, L, d_state); all the same io dtype (float32 or
    bfloat16).  A: (d_inner, d_state) float32; D, delta_bias: (d_inner,) float32; h0:
    (batch, d_inner, d_state) float32.  Returns out (and h_last when return_last_state).
    nseg: None = automatic time split (workspace sized and allocated here unless given), an int
    forces that many segments (ss_scan_fwd_ex).  zoh_exact: exact zero-order-hold input term
    (SS_FLAG_ZOH_EXACT, through ss_scan_fwd_ex).
    """
    batch, L, d_inner = u.shape
    d_state = B.shape[-1]
    code = _dtype_code(u)
    for name, t in (("u", u), ("delta", delta), ("z", z)):
        _dev(t, name, u.dtype, (batch, L, d_inner))
    for name, t in (("B", B), ("C", C)):
        _dev(t, name, u.dtype, (batch, L, d_state))
    _dev(A, "A", torch.float32, (d_inner, d_state))
    _dev(D, "D", torch.float32, (d_inner,))
    _dev(delta_bias, "delta_bias", torch.float32, (d_inner,))
    _dev(h0, "h0", torch.float32, (batch, d_inner, d_state))
    if out is None:
        out = torch.empty_like(u)
    _dev(out, "out", u.dtype, (batch, L, d_inner))
    if return_last_state and h_last is None:
        h_last = torch.empty((batch, d_inner, d_state), dtype=torch.float32, device=u.device)
    _dev(h_last, "h_last", torch.float32, (batch, d_inner, d_state))
    if workspace is None:
        nbytes = workspace_bytes(batch, L, d_inner, d_state, u.dtype, nseg)
        workspace = (torch.empty(nbytes, dtype=torch.uint8, device=u.device) if nbytes
                     else None)
    ws_ptr = _ptr(workspace)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            1 if delta_softplus else 0, _ptr(h0), _ptr(h_last), _ptr(out),
            batch, L, d_inner, d_state, code, ws_ptr, ws_len]
    if nseg is None and not zoh_exact:
        _check(lib().ss_scan_fwd(*args, _stream(stream)))
    else:
        flags = SS_FLAG_ZOH_EXACT if zoh_exact else 0
        _check(lib().ss_scan_fwd_ex(*args, int(nseg or 0), flags, _stream(stream)))
    return (out, h_last) if return_last_state else out


def scan_fwd_noalloc(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                     h0=None, out=None, h_last=None, stream=None):
    """Prefill through ss_scan_fwd_noalloc: the library allocates nothing and the time split,
    when used, keeps its carries in the library's static per-GPU scratch.  out (and h_last, if
    wanted) must be given: this call allocates nothing either.  Returns out."""
    batch, L, d_inner = u.shape
    d_state = B.shape[-1]
    code = _dtype_code(u)
    for name, t in (("u", u), ("delta", delta), ("z", z)):
        _dev(t, name, u.dtype, (batch, L, d_inner))
    for name, t in (("B", B), ("C", C)):
        _dev(t, name, u.dtype, (batch, L, d_state))
    _dev(A, "A", torch.float32, (d_inner, d_state))
    _dev(D, "D", torch.float32, (d_inner,))
    _dev(delta_bias, "delta_bias", torch.float32, (d_inner,))
    _dev(h0, "h0", torch.float32, (batch, d_inner, d_state))
    if out is None:
        raise ValueError("scan_fwd_noalloc: out must be given")
    _dev(out, "out", u.dtype, (batch, L, d_inner))
    _dev(h_last, "h_last", torch.float32, (batch, d_inner, d_state))
    _check(lib().ss_scan_fwd_noalloc(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
        1 if delta_softplus else 0, _ptr(h0), _ptr(h_last), _ptr(out), batch, L, d_inner,
        d_state, code, _stream(stream)))
    return out


def scan_fwd_conv(x, conv_weight, conv_bias, delta, A, B, C, D=None, z=None, delta_bias=None,
                  delta_softplus=True, x_prev=None, h0=None, return_last_state=False, out=None,
                  h_last=None, workspace=None, nseg=None, zoh_exact=False, stream=None):
    """Prefill with the fused front end (ss_scan_fwd_conv): u = silu(causal depthwise conv of x).

    x: (batch, L, d_inner) in the io dtype; conv_weight: (d_inner, k) float32, k in 1..4;
    conv_bias: (d_inner,) float32 or None; x_prev: (batch, k-1, d_inner) io dtype or None.  The
    rest as in scan_fwd.
    """
    batch, L, d_inner = x.shape
    d_state = B.shape[-1]
    code = _dtype_code(x)
    k = conv_weight.shape[-1]
    for name, t in (("x", x), ("delta", delta), ("z", z)):
        _dev(t, name, x.dtype, (batch, L, d_inner))
    for name, t in (("B", B), ("C", C)):
        _dev(t, name, x.dtype, (batch, L, d_state))
    _dev(conv_weight, "conv_weight", torch.float32, (d_inner, k))
    _dev(conv_bias, "conv_bias", torch.float32, (d_inner,))
    _dev(x_prev, "x_prev", x.dtype, (batch, k - 1, d_inner))
    _dev(A, "A", torch.float32, (d_inner, d_state))
    _dev(D, "D", torch.float32, (d_inner,))
    _dev(delta_bias, "delta_bias", torch.float32, (d_inner,))
    _dev(h0, "h0", torch.float32, (batch, d_inner, d_state))
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "out", x.dtype, (batch, L, d_inner))
    if return_last_state and h_last is None:
        h_last = torch.empty((batch, d_inner, d_state), dtype=torch.float32, device=x.device)
    _dev(h_last, "h_last", torch.float32, (batch, d_inner, d_state))
    if workspace is None:
        nbytes = workspace_bytes(batch, L, d_inner, d_state, x.dtype, nseg)
        workspace = (torch.empty(nbytes, dtype=torch.uint8, device=x.device) if nbytes
                     else None)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ss_scan_fwd_conv(
        _ptr(x), _ptr(conv_weight), _ptr(conv_bias), _ptr(x_prev), int(k), _ptr(delta), _ptr(A),
        _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), 1 if delta_softplus else 0,
        _ptr(h0), _ptr(h_last), _ptr(out), batch, L, d_inner, d_state, code, _ptr(workspace),
        ws_len, int(nseg or 0), SS_FLAG_ZOH_EXACT if zoh_exact else 0, _stream(stream)))
    return (out, h_last) if return_last_state else out


def scan_fwd_states(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                    h0=None, return_last_state=False, out=None, h_last=None, states=None,
                    workspace=None, stream=None):
    """Prefill that also saves the state after every 16-step chunk (ss_scan_fwd_states), for
    scan_bwd(..., states_given=True).  Arguments as for scan_fwd; states: (batch, ceil(L / 16),
    d_inner, d_state) float32 (the states view of bwd_workspace, to hand the workspace to the
    backward) or None (allocated here).  Returns (out, states), or (out, states, h_last) with
    return_last_state."""
    batch, L, d_inner = u.shape
    d_state = B.shape[-1]
    code = _dtype_code(u)
    for name, t in (("u", u), ("delta", delta), ("z", z)):
        _dev(t, name, u.dtype, (batch, L, d_inner))
    for name, t in (("B", B), ("C", C)):
        _dev(t, name, u.dtype, (batch, L, d_state))
    _dev(A, "A", torch.float32, (d_inner, d_state))
    _dev(D, "D", torch.float32, (d_inner,))
    _dev(delta_bias, "delta_bias", torch.float32, (d_inner,))
    _dev(h0, "h0", torch.float32, (batch, d_inner, d_state))
    if out is None:
        out = torch.empty_like(u)
    _dev(out, "out", u.dtype, (batch, L, d_inner))
    if return_last_state and h_last is None:
        h_last = torch.empty((batch, d_inner, d_state), dtype=torch.float32, device=u.device)
    _dev(h_last, "h_last", torch.float32, (batch, d_inner, d_state))
    nct = (L + 15) // 16
    if states is None:
        states = torch.empty((batch, nct, d_inner, d_state), dtype=torch.float32,
                             device=u.device)
    _dev(states, "states", torch.float32, (batch, nct, d_inner, d_state))
    if workspace is None:
        nbytes = workspace_bytes(batch, L, d_inner, d_state, u.dtype, None)
        workspace = (torch.empty(nbytes, dtype=torch.uint8, device=u.device) if nbytes
                     else None)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ss_scan_fwd_states(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
        1 if delta_softplus else 0, _ptr(h0), _ptr(h_last), _ptr(out), _ptr(states), batch, L,
        d_inner, d_state, code, _ptr(workspace), ws_len, _stream(stream)))
    return (out, states, h_last) if return_last_state else (out, states)


def bwd_workspace(batch, seqlen, d_inner, d_state, dtype=torch.bfloat16, device="cuda"):
    """A workspace for scan_bwd (ss_scan_bwd_workspace_bytes bytes, or None when it needs none)
    and the float32 view of its first part that holds the chunk-end states: give the view to
    scan_fwd_states(states=...) and the workspace to scan_bwd(..., states_given=True)."""
    code = SS_BF16 if dtype == torch.bfloat16 else SS_F32
    nbytes = int(lib().ss_scan_bwd_workspace_bytes(batch, seqlen, d_inner, d_state, code))
    if nbytes == 0:
        return None, None
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    nct = (seqlen + 15) // 16
    states = ws[:batch * nct * d_inner * d_state * 4].view(torch.float32).view(
        batch, nct, d_inner, d_state)
    return ws, states


def scan_bwd(u, delta, A, B, C, dout, D=None, z=None, delta_bias=None, delta_softplus=True,
             h0=None, dh_last=None, want_dD=True, want_ddelta_bias=True, want_dh0=True,
             workspace=None, states_given=False, zoh_exact=False, stream=None):
    """Gradients of scan_fwd (ss_scan_bwd) for the upstream gradient dout (same dtype and shape
    as out) and optionally dh_last.  Returns a dict: du, ddelta, dz (io dtype; dz None without
    z), dA, dB, dC (float32), dD, ddelta_bias, dh0 (float32, None when not wanted).
    workspace: uint8 device buffer of ss_scan_bwd_workspace_bytes bytes (allocated here when
    None).  states_given: the workspace already begins with the chunk-end states that
    scan_fwd_states saved for these inputs (SS_FLAG_STATES_GIVEN; see bwd_workspace), and the
    backward skips its own forward pass.  zoh_exact: gradients of the exact zero-order-hold
    input term (SS_FLAG_ZOH_EXACT; not with states_given)."""
    batch, L, d_inner = u.shape
    d_state = B.shape[-1]
    code = _dtype_code(u)
    for name, t in (("u", u), ("delta", delta), ("z", z), ("dout", dout)):
        _dev(t, name, u.dtype, (batch, L, d_inner))
    for name, t in (("B", B), ("C", C)):
        _dev(t, name, u.dtype, (batch, L, d_state))
    _dev(A, "A", torch.float32, (d_inner, d_state))
    _dev(D, "D", torch.float32, (d_inner,))
    _dev(delta_bias, "delta_bias", torch.float32, (d_inner,))
    _dev(h0, "h0", torch.float32, (batch, d_inner, d_state))
    _dev(dh_last, "dh_last", torch.float32, (batch, d_inner, d_state))
    f32 = dict(dtype=torch.float32, device=u.device)
    g = dict(du=torch.empty_like(u), ddelta=torch.empty_like(u),
             dz=torch.empty_like(u) if z is not None else None,
             dA=torch.empty((d_inner, d_state), **f32), dB=torch.empty((batch, L, d_state), **f32),
             dC=torch.empty((batch, L, d_state), **f32),
             dD=torch.empty((d_inner,), **f32) if want_dD else None,
             ddelta_bias=torch.empty((d_inner,), **f32) if want_ddelta_bias else None,
             dh0=torch.empty((batch, d_inner, d_state), **f32) if want_dh0 else None)
    flags = (SS_FLAG_STATES_GIVEN if states_given else 0) | (SS_FLAG_ZOH_EXACT if zoh_exact else 0)
    if workspace is None:
        if states_given:
            raise ValueError("states_given needs the workspace that holds the states")
        workspace, _ = bwd_workspace(batch, L, d_inner, d_state, u.dtype, u.device)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ss_scan_bwd(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
        1 if delta_softplus else 0, _ptr(h0), _ptr(dout), _ptr(dh_last), _ptr(g["du"]),
        _ptr(g["ddelta"]), _ptr(g["dz"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
        _ptr(g["dD"]), _ptr(g["ddelta_bias"]), _ptr(g["dh0"]), batch, L, d_inner, d_state, code,
        _ptr(workspace), ws_len, flags, _stream(stream)))
    return g


def scan2_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=True, h0=None,
              return_last_state=False, out=None, h_last=None, stream=None):
    """Multi-head scan with a scalar transition per head (ss_scan2_fwd).

    x, z: (batch, L, nheads, headdim); dt: (batch, L, nheads); B, C: (batch, L, ngroups,
    d_state), one io dtype.  A, D, dt_bias: (nheads,) float32.  h0: (batch, nheads, d_state,
    headdim) float32.  Returns out (and h_last when return_last_state).
    """
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    code = _dtype_code(x)
    for name, t in (("x", x), ("z", z)):
        _dev(t, name, x.dtype, (batch, L, H, P))
    _dev(dt, "dt", x.dtype, (batch, L, H))
    for name, t in (("B", B), ("C", C)):
        _dev(t, name, x.dtype, (batch, L, G, N))
    for name, t in (("A", A), ("D", D), ("dt_bias", dt_bias)):
        _dev(t, name, torch.float32, (H,))
    _dev(h0, "h0", torch.float32, (batch, H, N, P))
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "out", x.dtype, (batch, L, H, P))
    if return_last_state and h_last is None:
        h_last = torch.empty((batch, H, N, P), dtype=torch.float32, device=x.device)
    _dev(h_last, "h_last", torch.float32, (batch, H, N, P))
    _check(lib().ss_scan2_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                              _ptr(dt_bias), 1 if dt_softplus else 0, _ptr(h0), _ptr(h_last),
                              _ptr(out), batch, L, H, P, G, N, code, _stream(stream)))
    return (out, h_last) if return_last_state else out


def state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None,
                 delta_softplus=True, out=None, zoh_exact=False, stream=None):
    """One decode step on the GPU (ss_state_update); `state` is updated in place.

    state: (batch, d_inner, d_state) float32; u, delta, z: (batch, d_inner); B, C:
    (batch, d_state) in the io dtype.  Returns out: (batch, d_inner).
    """
    batch, d_inner, d_state = state.shape
    code = _dtype_code(u)
    _dev(state, "state", torch.float32)
    for name, t in (("u", u), ("delta", delta), ("z", z)):
        _dev(t, name, u.dtype, (batch, d_inner))
    for name, t in (("B", B), ("C", C)):
        _dev(t, name, u.dtype, (batch, d_state))
    _dev(A, "A", torch.float32, (d_inner, d_state))
    _dev(D, "D", torch.float32, (d_inner,))
    _dev(delta_bias, "delta_bias", torch.float32, (d_inner,))
    if out is None:
        out = torch.empty_like(u)
    _dev(out, "out", u.dtype, (batch, d_inner))
    args = [_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(delta_bias), 1 if delta_softplus else 0, _ptr(out), batch, d_inner, d_state, code]
    if zoh_exact:
        _check(lib().ss_state_update_ex(*args, SS_FLAG_ZOH_EXACT, _stream(stream)))
    else:
        _check(lib().ss_state_update(*args, _stream(stream)))
    return out


def state_update_conv(state, conv_state, x, conv_weight, conv_bias, delta, A, B, C, D=None,
                      z=None, delta_bias=None, delta_softplus=True, out=None, zoh_exact=False,
                      stream=None):
    """One decode step with the fused front end (ss_state_update_conv): state (batch, d_inner,
    d_state) float32 and conv_state (batch, k-1, d_inner) io dtype are updated in place; x,
    delta, z: (batch, d_inner); conv_weight (d_inner, k) float32; conv_bias (d_inner,) or None."""
    batch, d_inner, d_state = state.shape
    code = _dtype_code(x)
    k = conv_weight.shape[-1]
    _dev(state, "state", torch.float32)
    _dev(conv_state, "conv_state", x.dtype, (batch, k - 1, d_inner))
    for name, t in (("x", x), ("delta", delta), ("z", z)):
        _dev(t, name, x.dtype, (batch, d_inner))
    for name, t in (("B", B), ("C", C)):
        _dev(t, name, x.dtype, (batch, d_state))
    _dev(conv_weight, "conv_weight", torch.float32, (d_inner, k))
    _dev(conv_bias, "conv_bias", torch.float32, (d_inner,))
    _dev(A, "A", torch.float32, (d_inner, d_state))
    _dev(D, "D", torch.float32, (d_inner,))
    _dev(delta_bias, "delta_bias", torch.float32, (d_inner,))
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "out", x.dtype, (batch, d_inner))
    _check(lib().ss_state_update_conv(
        _ptr(state), _ptr(conv_state), _ptr(x), _ptr(conv_weight), _ptr(conv_bias), int(k),
        _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
        1 if delta_softplus else 0, _ptr(out), batch, d_inner, d_state, code,
        SS_FLAG_ZOH_EXACT if zoh_exact else 0, _stream(stream)))
    return out
