"""fp64 CPU reference ("oracle") for the selective state-space scan (S6).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The GPU library never imports, links or calls it,
and the two share no code.

The arithmetic lives in ``ss_oracle.c`` (plain C, IEEE double, sequential in time); this module
only builds it with gcc and marshals numpy arrays into it.  ``numpy_twin`` holds an independent
pure-numpy transcription used on tiny inputs to cross-check the C build.

Sources: the Mamba reading guide (xyznot.com), sections "Método" and "O Mecanismo de Seleção
(S6)"; the IBM explainer "O que é um modelo Mamba?" (state/output equations, Mamba block); the
aivaro.ru answer "Как работает Mamba", section 3 "Selective Scan".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ss_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libss_oracle.so")

F32, BF16, F64 = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile ss_oracle.c into libss_oracle.so next to it (gcc, -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-Wall", "-Werror",
             "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def use_library(path):
    """Point this module at another build of ss_oracle.c (used by the mutation tests, which
    compile deliberately broken copies and check that the pins catch them).  Returns the previous
    handle so that it can be restored with restore_library()."""
    global _lib
    prev = _lib
    _lib = _bind(ctypes.CDLL(path))
    return prev


def restore_library(prev):
    global _lib
    _lib = prev


def _bind(lib):
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_scan_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32,
                                    i64, i64, i64, i64, vp, i64, vp, vp, i32]
    lib.oracle_scan_fwd.restype = i32
    lib.oracle_scan_fwd_chunked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32,
                                            i32, i64, i64, i64, i64, i64, vp, vp]
    lib.oracle_scan_fwd_chunked.restype = i32
    lib.oracle_state_update.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                        i32, i64, i64, i64, vp, i64, vp, i32]
    lib.oracle_conv_silu.argtypes = [vp, vp, vp, vp, i64, i32, i64, i64, i64, vp]
    lib.oracle_conv_silu.restype = i32
    lib.oracle_scan_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i64, i64,
                                    i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32]
    lib.oracle_scan_bwd.restype = i32
    lib.oracle_scan2_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i64, i64, i64,
                                     i64, i64, i64, vp, vp, i32]
    lib.oracle_scan2_fwd.restype = i32
    lib.oracle_state_update.restype = i32
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i32
    return lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _io(x, name):
    """Accept float32 arrays, or bf16 given as raw uint16 bit patterns."""
    if x is None:
        return None, None
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError(f"{name}: expected float32 or uint16 (bf16 bits), got {x.dtype}")


def _io_u(u, io_dtype):
    """u in the io dtype, or float64 (the output of conv_silu)."""
    if isinstance(u, np.ndarray) and u.dtype == np.float64:
        return np.ascontiguousarray(u), F64
    u, dt = _io(u, "u")
    if dt != io_dtype:
        raise TypeError("u: io dtype differs from delta's")
    return u, dt


def _f32(x, shape, name):
    if x is None:
        return None
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.shape != shape:
        raise ValueError(f"{name}: shape {x.shape}, expected {shape}")
    return x


def _ptr(x):
    return None if x is None else x.ctypes.data


def _check_io(arrs, shapes, dtype_ref):
    for (name, a), shp in zip(arrs, shapes):
        if a is None:
            continue
        if a.shape != shp:
            raise ValueError(f"{name}: shape {a.shape}, expected {shp}")
        if (a.dtype == np.uint16) != (dtype_ref == BF16):
            raise TypeError(f"{name}: io dtype differs from u's")


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
             h0=None, zoh_exact=False, rows=None, nthreads=None):
    """Sequential fp64 prefill.

    u, delta, z: (batch, L, d_inner); B, C: (batch, L, d_state) -- float32, or uint16 holding
    bf16 bits (all five in the same io dtype).  A: (d_inner, d_state); D, delta_bias: (d_inner,).
    h0: (batch, d_inner, d_state) float64 or None.  rows: optional 1-D array of row ids
    b*d_inner + d.

    u may instead be float64 (the unrounded output of conv_silu).

    Returns (out, h_last): without rows, out is (batch, L, d_inner) and h_last is
    (batch, d_inner, d_state); with rows, out is (len(rows), L) and h_last (len(rows), d_state).
    """
    delta, dt = _io(delta, "delta")
    u, udt = _io_u(u, dt)
    B, _ = _io(B, "B")
    C, _ = _io(C, "C")
    z, _ = _io(z, "z")
    batch, L, d_inner = u.shape
    d_state = B.shape[2]
    _check_io([("delta", delta), ("z", z), ("B", B), ("C", C)],
              [(batch, L, d_inner), (batch, L, d_inner), (batch, L, d_state),
               (batch, L, d_state)], dt)
    A = _f32(A, (d_inner, d_state), "A")
    D = _f32(D, (d_inner,), "D")
    delta_bias = _f32(delta_bias, (d_inner,), "delta_bias")
    if h0 is not None:
        h0 = np.ascontiguousarray(h0, dtype=np.float64).reshape(batch, d_inner, d_state)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows.shape[0]
    else:
        nrows = batch * d_inner
    out = np.empty((nrows, L), dtype=np.float64)
    h_last = np.empty((nrows, d_state), dtype=np.float64)
    if nthreads is None:
        nthreads = max(1, len(os.sched_getaffinity(0)))
    rc = _load().oracle_scan_fwd(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
        int(bool(delta_softplus)), _ptr(h0), int(bool(zoh_exact)), dt, udt,
        batch, L, d_inner, d_state, _ptr(rows), nrows, _ptr(out), _ptr(h_last), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_scan_fwd rejected its arguments")
    if rows is None:
        out = out.reshape(batch, d_inner, L).transpose(0, 2, 1)
        h_last = h_last.reshape(batch, d_inner, d_state)
    return out, h_last


def scan_fwd_chunked(u, delta, A, B, C, chunk, D=None, z=None, delta_bias=None,
                     delta_softplus=True, h0=None, zoh_exact=False):
    """Same result as scan_fwd via the blockwise associative decomposition (block = chunk)."""
    delta, dt = _io(delta, "delta")
    u, udt = _io_u(u, dt)
    B, _ = _io(B, "B")
    C, _ = _io(C, "C")
    z, _ = _io(z, "z")
    batch, L, d_inner = u.shape
    d_state = B.shape[2]
    _check_io([("delta", delta), ("z", z), ("B", B), ("C", C)],
              [(batch, L, d_inner), (batch, L, d_inner), (batch, L, d_state),
               (batch, L, d_state)], dt)
    A = _f32(A, (d_inner, d_state), "A")
    D = _f32(D, (d_inner,), "D")
    delta_bias = _f32(delta_bias, (d_inner,), "delta_bias")
    if h0 is not None:
        h0 = np.ascontiguousarray(h0, dtype=np.float64).reshape(batch, d_inner, d_state)
    out = np.empty((batch * d_inner, L), dtype=np.float64)
    h_last = np.empty((batch * d_inner, d_state), dtype=np.float64)
    rc = _load().oracle_scan_fwd_chunked(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
        int(bool(delta_softplus)), _ptr(h0), int(bool(zoh_exact)), dt, udt,
        batch, L, d_inner, d_state, int(chunk), _ptr(out), _ptr(h_last))
    if rc != 0:
        raise ValueError("oracle_scan_fwd_chunked rejected its arguments")
    return (out.reshape(batch, d_inner, L).transpose(0, 2, 1),
            h_last.reshape(batch, d_inner, d_state))


def state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None,
                 delta_softplus=True, zoh_exact=False, rows=None, nthreads=None):
    """One fp64 decode step.  state: (batch, d_inner, d_state) float64, updated IN PLACE (only
    the selected rows when rows is given).  u, delta, z: (batch, d_inner); B, C:
    (batch, d_state).  Returns out: (batch, d_inner), or (len(rows),) with rows."""
    if not (isinstance(state, np.ndarray) and state.dtype == np.float64
            and state.flags.c_contiguous):
        raise TypeError("state must be a C-contiguous float64 array (updated in place)")
    delta, dt = _io(delta, "delta")
    u, udt = _io_u(u, dt)
    B, _ = _io(B, "B")
    C, _ = _io(C, "C")
    z, _ = _io(z, "z")
    batch, d_inner = u.shape
    d_state = B.shape[1]
    if state.shape != (batch, d_inner, d_state):
        raise ValueError(f"state: shape {state.shape}, expected {(batch, d_inner, d_state)}")
    _check_io([("delta", delta), ("z", z), ("B", B), ("C", C)],
              [(batch, d_inner), (batch, d_inner), (batch, d_state), (batch, d_state)], dt)
    A = _f32(A, (d_inner, d_state), "A")
    D = _f32(D, (d_inner,), "D")
    delta_bias = _f32(delta_bias, (d_inner,), "delta_bias")
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows.shape[0]
    else:
        nrows = batch * d_inner
    out = np.empty((nrows,), dtype=np.float64)
    if nthreads is None:
        nthreads = max(1, len(os.sched_getaffinity(0)))
    rc = _load().oracle_state_update(
        _ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
        _ptr(delta_bias), int(bool(delta_softplus)), int(bool(zoh_exact)), dt, udt,
        batch, d_inner, d_state, _ptr(rows), nrows, _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_state_update rejected its arguments")
    return out.reshape(batch, d_inner) if rows is None else out


def conv_silu(x, w, b=None, x_prev=None):
    """The block's front end in fp64: u = silu(causal depthwise conv of x + b), see
    oracle_conv_silu in ss_oracle.c.  x: (batch, L, d_inner) float32 or bf16 bits; w:
    (d_inner, k) float32; b: (d_inner,) float32 or None; x_prev: (batch, k-1, d_inner) in x's
    dtype (the inputs before t = 0) or None for zeros.  Returns u: (batch, L, d_inner) float64."""
    x, dt = _io(x, "x")
    batch, L, d_inner = x.shape
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[0] != d_inner:
        raise ValueError(f"w: shape {w.shape}, expected ({d_inner}, k)")
    k = w.shape[1]
    b = _f32(b, (d_inner,), "b")
    if x_prev is not None:
        x_prev, pdt = _io(x_prev, "x_prev")
        if pdt != dt or x_prev.shape != (batch, k - 1, d_inner):
            raise ValueError(f"x_prev: expected {(batch, k - 1, d_inner)} in x's dtype")
    u = np.empty((batch, L, d_inner), dtype=np.float64)
    rc = _load().oracle_conv_silu(_ptr(x), _ptr(w), _ptr(b), _ptr(x_prev), k, dt, batch, L,
                                  d_inner, _ptr(u))
    if rc != 0:
        raise ValueError("oracle_conv_silu rejected its arguments")
    return u


def conv_step(conv_state, x, w, b=None):
    """One decode step of the front end: conv_state (batch, k-1, d_inner) holds the k-1 previous
    inputs (oldest first), x (batch, d_inner) the new one.  Returns (u float64 (batch, d_inner),
    the new conv_state): the window shifted by one with x appended."""
    x = np.ascontiguousarray(x)
    u = conv_silu(x[:, None, :], w, b, x_prev=conv_state)[:, 0, :]
    new_state = np.concatenate([conv_state, x[:, None, :]], axis=1)[:, 1:, :]
    return u, np.ascontiguousarray(new_state)


def scan_bwd(u, delta, A, B, C, dout, D=None, z=None, delta_bias=None, delta_softplus=True,
             h0=None, dh_last=None, zoh_exact=False, nthreads=None):
    """fp64 gradients of scan_fwd (first-order input term, or the exact ZOH one with zoh_exact)
    for upstream gradients dout (batch, L, d_inner) and dh_last (batch, d_inner, d_state) or
    None.  Inputs as for scan_fwd (u in the io dtype).  Returns a dict with du, ddelta, dz (None
    without z), dA, dB, dC, dD, ddelta_bias, dh0 -- float64 arrays shaped like the
    corresponding inputs.  Rows run on nthreads OpenMP threads (default: every core this
    process may use); the sums over rows are added in a fixed order for a given count."""
    delta, dt = _io(delta, "delta")
    u, udt = _io_u(u, dt)
    if udt != dt:
        raise TypeError("scan_bwd takes u in the io dtype")
    B, _ = _io(B, "B")
    C, _ = _io(C, "C")
    z, _ = _io(z, "z")
    batch, L, d_inner = u.shape
    d_state = B.shape[2]
    _check_io([("delta", delta), ("z", z), ("B", B), ("C", C)],
              [(batch, L, d_inner), (batch, L, d_inner), (batch, L, d_state),
               (batch, L, d_state)], dt)
    A = _f32(A, (d_inner, d_state), "A")
    D = _f32(D, (d_inner,), "D")
    delta_bias = _f32(delta_bias, (d_inner,), "delta_bias")
    if h0 is not None:
        h0 = np.ascontiguousarray(h0, dtype=np.float64).reshape(batch, d_inner, d_state)
    dout = np.ascontiguousarray(dout, dtype=np.float64).reshape(batch, L, d_inner)
    if dh_last is not None:
        dh_last = np.ascontiguousarray(dh_last, dtype=np.float64).reshape(batch, d_inner, d_state)
    g = dict(du=np.empty((batch, L, d_inner)), ddelta=np.empty((batch, L, d_inner)),
             dz=np.empty((batch, L, d_inner)) if z is not None else None,
             dA=np.empty((d_inner, d_state)), dB=np.empty((batch, L, d_state)),
             dC=np.empty((batch, L, d_state)), dD=np.empty(d_inner),
             ddelta_bias=np.empty(d_inner), dh0=np.empty((batch, d_inner, d_state)))
    if nthreads is None:
        nthreads = max(1, len(os.sched_getaffinity(0)))
    rc = _load().oracle_scan_bwd(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
        int(bool(delta_softplus)), _ptr(h0), int(bool(zoh_exact)), dt, batch, L, d_inner,
        d_state, _ptr(dout), _ptr(dh_last), _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dz"]),
        _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["ddelta_bias"]),
        _ptr(g["dh0"]), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_scan_bwd rejected its arguments")
    return g


def scan2_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=True, h0=None,
              nthreads=None):
    """Sequential fp64 multi-head scan with a scalar transition per head (oracle_scan2_fwd).
    x, z: (batch, L, nheads, headdim); dt: (batch, L, nheads); B, C: (batch, L, ngroups,
    d_state) -- float32 or bf16 bits, one io dtype.  A, D, dt_bias: (nheads,) float32.  h0:
    (batch, nheads, d_state, headdim) float64 or None.  Returns (out, h_last) in float64."""
    x, io = _io(x, "x")
    dt, _ = _io(dt, "dt")
    B, _ = _io(B, "B")
    C, _ = _io(C, "C")
    z, _ = _io(z, "z")
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _check_io([("dt", dt), ("z", z), ("B", B), ("C", C)],
              [(batch, L, H), (batch, L, H, P), (batch, L, G, N), (batch, L, G, N)], io)
    A = _f32(A, (H,), "A")
    D = _f32(D, (H,), "D")
    dt_bias = _f32(dt_bias, (H,), "dt_bias")
    if h0 is not None:
        h0 = np.ascontiguousarray(h0, dtype=np.float64).reshape(batch, H, N, P)
    out = np.empty((batch, L, H, P))
    h_last = np.empty((batch, H, N, P))
    if nthreads is None:
        nthreads = max(1, len(os.sched_getaffinity(0)))
    rc = _load().oracle_scan2_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                  _ptr(dt_bias), int(bool(dt_softplus)), _ptr(h0), io, batch, L,
                                  H, P, G, N, _ptr(out), _ptr(h_last), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_scan2_fwd rejected its arguments")
    return out, h_last
