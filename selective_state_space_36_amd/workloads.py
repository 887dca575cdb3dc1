"""Seeded synthetic inputs for the selective scan (S6) workloads.

This module only draws random numbers and rounds them to the input dtype; it holds none of the
scan's arithmetic.  Both the GPU path and the fp64 reference consume its arrays, so the two are
always compared on identical input bytes.

Shapes follow the Mamba layer statement: u, delta, z of shape (batch, L, d_inner); B and C of
shape (batch, L, d_state) shared by all channels; a real diagonal A of shape (d_inner, d_state);
a per-channel skip D and a per-channel step-size bias.  The sizes (Mamba-130M- and
Mamba-2.8B-shaped layers, a million-step sequence, a batch-128 decode step) are the synthetic
stand-ins for real activations; no dataset or trained weight is involved.

Recipe (all draws from numpy PCG64):
  * seed = 1000 + workload index; SeedSequence(seed).spawn(8) gives one child per tensor in the
    fixed order u, delta, z, B, C, dt, D, h0/state; each child is split again into one stream per
    2**26-element chunk so that large tensors are drawn by several threads.
  * u, delta (raw), z, B, C ~ N(0, 1) (delta is 0.5 * N(0, 1) in the tiny fp32 case), drawn in
    float32 and rounded to bf16 with round-to-nearest-even where the io dtype is bf16.
  * per-channel step size dt ~ log-uniform[lo, hi]; delta_bias = log(expm1(dt)), i.e. the bias
    whose softplus is dt, so that softplus(delta_raw + bias) is spread around dt.
  * A[d, n] = -(n + 1) (S4D-real), float32.
  * D = 1 (tiny case) or ~ N(1, 0.1) (std 0.1), float32.
  * decode: resident state ~ N(0, 1) float32; every step draws fresh u, delta, z, B, C.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 26


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    batch: int
    seqlen: int          # time steps per call (1 for decode)
    d_inner: int
    d_state: int
    io_dtype: str        # "f32" or "bf16"
    gate: bool
    dt_lo: float
    dt_hi: float
    delta_scale: float   # std of the raw delta draw
    d_skip: str          # "one" or "normal"
    decode_steps: int = 0

    @property
    def elements(self) -> int:
        return self.batch * self.seqlen * self.d_inner

    @property
    def is_decode(self) -> bool:
        return self.decode_steps > 0


WORKLOADS = {
    0: Workload(0, "tiny-fp32", 1, 128, 64, 16, "f32", False, 1e-3, 1e-1, 0.5, "one"),
    1: Workload(1, "mamba130m-prefill", 8, 2048, 1536, 16, "bf16", True, 1e-3, 1e-1, 1.0,
                "normal"),
    2: Workload(2, "mamba2.8b-prefill", 4, 4096, 5120, 16, "bf16", True, 1e-3, 1e-1, 1.0,
                "normal"),
    3: Workload(3, "long-1M-prefill", 1, 1 << 20, 1536, 16, "bf16", True, 1e-4, 1e-2, 1.0,
                "normal"),
    4: Workload(4, "decode-b128", 128, 1, 5120, 16, "bf16", True, 1e-3, 1e-1, 1.0, "normal",
                decode_steps=1000),
}


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (round-to-nearest-even); returns the uint16 bits."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(bits.shape, dtype=np.uint16)
    flat_in, flat_out = bits.reshape(-1), out.reshape(-1)

    def work(lo, hi):
        b = flat_in[lo:hi]
        r = (b >> np.uint32(16)) & np.uint32(1)
        flat_out[lo:hi] = ((b + np.uint32(0x7FFF) + r) >> np.uint32(16)).astype(np.uint16)

    _chunked(flat_in.size, work)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _chunked(n, fn):
    spans = [(lo, min(n, lo + CHUNK)) for lo in range(0, n, CHUNK)]
    if len(spans) <= 1:
        for lo, hi in spans:
            fn(lo, hi)
        return
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda s: fn(*s), spans))


def normal_f32(seq: np.random.SeedSequence, shape, scale=1.0, loc=0.0) -> np.ndarray:
    """float32 N(loc, scale^2) draws; chunk k of 2**26 elements uses seq.spawn(...)[k]."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    kids = seq.spawn(max(1, -(-n // CHUNK)))

    def work(lo, hi):
        g = np.random.Generator(np.random.PCG64(kids[lo // CHUNK]))
        g.standard_normal(out=out[lo:hi], dtype=np.float32)
        if scale != 1.0:
            out[lo:hi] *= np.float32(scale)
        if loc != 0.0:
            out[lo:hi] += np.float32(loc)

    _chunked(n, work)
    return out.reshape(shape)


def _io_cast(x: np.ndarray, io_dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if io_dtype == "bf16" else x


def _params(w: Workload, kids, d_inner: int):
    """A, D and delta_bias for a workload (float32)."""
    g_dt = np.random.Generator(np.random.PCG64(kids[5]))
    dt = np.exp(g_dt.uniform(np.log(w.dt_lo), np.log(w.dt_hi), size=d_inner))
    delta_bias = np.log(np.expm1(dt)).astype(np.float32)
    A = np.tile(-np.arange(1, w.d_state + 1, dtype=np.float32), (d_inner, 1))
    if w.d_skip == "one":
        D = np.ones(d_inner, dtype=np.float32)
    else:
        D = normal_f32(kids[6], (d_inner,), scale=0.1, loc=1.0)
    return np.ascontiguousarray(A), D, delta_bias


def make_prefill(w: Workload, *, batch=None, seqlen=None, d_inner=None, seed=None):
    """Inputs for a prefill workload (sizes may be overridden for smaller test cases).

    Returns a dict with u, delta, z (None without gate), B, C in the io dtype (float32 arrays,
    or uint16 bf16 bits) and A, D, delta_bias in float32.
    """
    if w.is_decode:
        raise ValueError("use make_decode for the decode workload")
    batch = w.batch if batch is None else batch
    seqlen = w.seqlen if seqlen is None else seqlen
    d_inner = w.d_inner if d_inner is None else d_inner
    seed = 1000 + w.index if seed is None else seed
    kids = np.random.SeedSequence(seed).spawn(8)
    x_shape = (batch, seqlen, d_inner)
    bc_shape = (batch, seqlen, w.d_state)
    u = _io_cast(normal_f32(kids[0], x_shape), w.io_dtype)
    delta = _io_cast(normal_f32(kids[1], x_shape, scale=w.delta_scale), w.io_dtype)
    z = _io_cast(normal_f32(kids[2], x_shape), w.io_dtype) if w.gate else None
    B = _io_cast(normal_f32(kids[3], bc_shape), w.io_dtype)
    C = _io_cast(normal_f32(kids[4], bc_shape), w.io_dtype)
    A, D, delta_bias = _params(w, kids, d_inner)
    return dict(u=u, delta=delta, z=z, B=B, C=C, A=A, D=D, delta_bias=delta_bias)


def make_decode(w: Workload, *, steps=None, batch=None, d_inner=None, seed=None):
    """Inputs for the decode workload: a float32 initial state (batch, d_inner, d_state), and per
    step u, delta, z of shape (steps, batch, d_inner) and B, C of shape (steps, batch, d_state),
    in the io dtype, plus A, D, delta_bias."""
    if not w.is_decode:
        raise ValueError("not a decode workload")
    steps = w.decode_steps if steps is None else steps
    batch = w.batch if batch is None else batch
    d_inner = w.d_inner if d_inner is None else d_inner
    seed = 1000 + w.index if seed is None else seed
    kids = np.random.SeedSequence(seed).spawn(8)
    x_shape = (steps, batch, d_inner)
    bc_shape = (steps, batch, w.d_state)
    u = _io_cast(normal_f32(kids[0], x_shape), w.io_dtype)
    delta = _io_cast(normal_f32(kids[1], x_shape, scale=w.delta_scale), w.io_dtype)
    z = _io_cast(normal_f32(kids[2], x_shape), w.io_dtype) if w.gate else None
    B = _io_cast(normal_f32(kids[3], bc_shape), w.io_dtype)
    C = _io_cast(normal_f32(kids[4], bc_shape), w.io_dtype)
    A, D, delta_bias = _params(w, kids, d_inner)
    state = normal_f32(kids[7], (batch, d_inner, w.d_state))
    return dict(state=state, u=u, delta=delta, z=z, B=B, C=C, A=A, D=D, delta_bias=delta_bias)


@dataclasses.dataclass(frozen=True)
class MultiHeadWorkload:
    """A layer of the multi-head scalar-transition scan (the Mamba-2 form)."""
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    ngroups: int
    d_state: int
    io_dtype: str
    gate: bool
    seed: int

    @property
    def elements(self) -> int:
        return self.batch * self.seqlen * self.nheads * self.headdim


# d_inner 5120 as 80 heads of 64 channels, one group of B/C with 128 states: the Mamba-2-shaped
# counterpart of the 2.8B prefill layer.
MULTIHEAD = MultiHeadWorkload("mamba2-80h-prefill", batch=4, seqlen=4096, nheads=80, headdim=64,
                              ngroups=1, d_state=128, io_dtype="bf16", gate=True, seed=2000)


def make_multihead(w: MultiHeadWorkload, *, batch=None, seqlen=None, nheads=None, headdim=None,
                   ngroups=None, d_state=None, seed=None):
    """Inputs for the multi-head scan: x, z (batch, L, H, P), dt (batch, L, H), B, C
    (batch, L, G, N) in the io dtype, and per head A = -U[1, 16], D ~ N(1, 0.1) and dt_bias with
    softplus(dt_bias) ~ log-uniform[1e-3, 1e-1] (float32).  Same stream discipline as
    make_prefill: SeedSequence(seed).spawn(8) in the order x, dt, z, B, C, dt-range, D, A."""
    batch = w.batch if batch is None else batch
    seqlen = w.seqlen if seqlen is None else seqlen
    H = w.nheads if nheads is None else nheads
    P = w.headdim if headdim is None else headdim
    G = w.ngroups if ngroups is None else ngroups
    N = w.d_state if d_state is None else d_state
    seed = w.seed if seed is None else seed
    kids = np.random.SeedSequence(seed).spawn(8)
    x = _io_cast(normal_f32(kids[0], (batch, seqlen, H, P)), w.io_dtype)
    dt = _io_cast(normal_f32(kids[1], (batch, seqlen, H), scale=0.5), w.io_dtype)
    z = _io_cast(normal_f32(kids[2], (batch, seqlen, H, P)), w.io_dtype) if w.gate else None
    B = _io_cast(normal_f32(kids[3], (batch, seqlen, G, N)), w.io_dtype)
    C = _io_cast(normal_f32(kids[4], (batch, seqlen, G, N)), w.io_dtype)
    g_dt = np.random.Generator(np.random.PCG64(kids[5]))
    dts = np.exp(g_dt.uniform(np.log(1e-3), np.log(1e-1), size=H))
    dt_bias = np.log(np.expm1(dts)).astype(np.float32)
    D = normal_f32(kids[6], (H,), scale=0.1, loc=1.0)
    g_a = np.random.Generator(np.random.PCG64(kids[7]))
    A = (-g_a.uniform(1.0, 16.0, size=H)).astype(np.float32)
    return dict(x=x, dt=dt, z=z, B=B, C=C, A=A, D=D, dt_bias=dt_bias)
