"""GPU checks of the saved chunk-end states (ss_scan_fwd_states) and of the backward that takes
them (ss_scan_bwd with SS_FLAG_STATES_GIVEN): each saved state equals the fp64 oracle's final
state of the prefix ending at that chunk, the forward's outputs are the plain forward's, and the
backward's gradients with given states match both the oracle and the backward that recomputes
them."""
import numpy as np
import pytest

import oracle
from selective_state_space_36_amd import workloads as wl
from tests.helpers import TOL, Errors, check_close, dev, host
from tests.test_gpu_bwd import check_grad, wl_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selective_state_space_36_amd import ops
    ops.lib()
    yield


def ops():
    from selective_state_space_36_amd import ops as o
    return o


def prefix(p, n):
    return {k: (np.ascontiguousarray(v[:, :n])
                if k in ("u", "delta", "z", "B", "C") and v is not None else v)
            for k, v in p.items()}


def check_states(p, h0, *, gate=True):
    batch, L, D = p["u"].shape
    N = p["B"].shape[-1]
    z = p["z"] if gate else None
    print(f"  states case: shape={p['u'].shape} N={N} dtype={p['u'].dtype} h0={h0 is not None}",
          flush=True)
    args = (dev(p["u"]), dev(p["delta"]), dev(p["A"]), dev(p["B"]), dev(p["C"]))
    kw = dict(D=dev(p["D"]), z=dev(z), delta_bias=dev(p["delta_bias"]),
              h0=None if h0 is None else dev(h0))
    out_s, states, hl = ops().scan_fwd_states(*args, return_last_state=True, **kw)
    out_p, hl_p = ops().scan_fwd(*args, return_last_state=True, **kw)
    torch.cuda.synchronize()
    # saving the states does not change the outputs
    assert torch.equal(out_s, out_p) and torch.equal(hl, hl_p)
    nct = (L + 15) // 16
    assert tuple(states.shape) == (batch, nct, D, N)
    st = host(states)
    check_close(st[:, -1, :, :], host(hl), 0.0, "last saved state == h_last")
    for c in sorted({0, 1, nct // 2, nct - 2, nct - 1} & set(range(nct))):
        n = min(16 * (c + 1), L)
        q = prefix(p, n)
        _, ref_h = oracle.scan_fwd(q["u"], q["delta"], q["A"], q["B"], q["C"], D=q["D"],
                                   z=q["z"] if gate else None, delta_bias=q["delta_bias"],
                                   h0=None if h0 is None else h0.astype(np.float64))
        check_close(st[:, c, :, :], ref_h, TOL["f32"], f"state after chunk {c} (step {n - 1})")
    return states


@pytest.mark.parametrize("L,N", [(1, 16), (16, 16), (70, 16), (100, 5), (45, 40)])
def test_saved_states_fp32(L, N):
    p = wl.make_prefill(wl.WORKLOADS[0], batch=2, seqlen=L, d_inner=24, seed=L + N)
    rng = np.random.default_rng(L)
    if N != 16:
        p["B"] = rng.standard_normal((2, L, N)).astype(np.float32)
        p["C"] = rng.standard_normal((2, L, N)).astype(np.float32)
        p["A"] = np.ascontiguousarray(np.tile(-np.arange(1, N + 1, dtype=np.float32), (24, 1)))
    h0 = rng.standard_normal((2, 24, N)).astype(np.float32)
    check_states(p, h0, gate=False)


def test_saved_states_bf16_time_split():
    """Few channels and a long sequence: the forward splits time into segments, and the states
    saved by later segments start from the carried state."""
    p = wl.make_prefill(wl.WORKLOADS[1], batch=1, seqlen=6000, d_inner=32, seed=3)
    ws = ops().workspace_bytes(1, 6000, 32, 16, torch.bfloat16)
    assert ws > 0  # the automatic split is active for this shape
    check_states(p, None)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_backward_with_saved_states(io):
    w = wl.WORKLOADS[0] if io == "f32" else wl.WORKLOADS[1]
    p = wl.make_prefill(w, batch=2, seqlen=150, d_inner=48, seed=7)
    rng = np.random.default_rng(8)
    batch, L, D = p["u"].shape
    N = p["B"].shape[-1]
    g_out = rng.standard_normal((batch, L, D)).astype(np.float32)
    if io == "bf16":
        g_out = wl.f32_to_bf16_bits(g_out)
    h0 = rng.standard_normal((batch, D, N)).astype(np.float32)
    z = p["z"] if w.gate else None
    args = (dev(p["u"]), dev(p["delta"]), dev(p["A"]), dev(p["B"]), dev(p["C"]))
    kw = dict(D=dev(p["D"]), z=dev(z), delta_bias=dev(p["delta_bias"]), h0=dev(h0))
    ws, states = ops().bwd_workspace(batch, L, D, N, args[0].dtype)
    ops().scan_fwd_states(*args, states=states, **kw)
    g_s = ops().scan_bwd(*args, dev(g_out), workspace=ws, states_given=True, **kw)
    g_r = ops().scan_bwd(*args, dev(g_out), **kw)
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], wl_f64(g_out), D=p["D"],
                          z=z, delta_bias=p["delta_bias"], h0=h0.astype(np.float64))
    io_tol = 2e-2 if io == "bf16" else 1e-3
    for key in ("du", "ddelta", "dz"):
        if ref[key] is None:
            continue
        check_grad(host(g_s[key]), ref[key], io_tol, key + " (given states)")
        check_grad(host(g_s[key]), host(g_r[key]), io_tol, key + " (given vs recomputed)")
    for key in ("dA", "dB", "dC", "dD", "ddelta_bias", "dh0"):
        check_grad(host(g_s[key]), ref[key], 1e-3, key + " (given states)")
        check_grad(host(g_s[key]), host(g_r[key]), 1e-4, key + " (given vs recomputed)")


def test_saved_states_full_size_every_row():
    """The 2.8B-shaped layer in the benchmark's configuration: the saved states of every row
    after three chunks against the oracle's prefix scans."""
    w = wl.WORKLOADS[2]
    p = wl.make_prefill(w)
    _, states = ops().scan_fwd_states(dev(p["u"]), dev(p["delta"]), dev(p["A"]), dev(p["B"]),
                                      dev(p["C"]), D=dev(p["D"]), z=dev(p["z"]),
                                      delta_bias=dev(p["delta_bias"]))
    torch.cuda.synchronize()
    for c in (0, 100, 255):
        q = prefix(p, 16 * (c + 1))
        _, ref_h = oracle.scan_fwd(q["u"], q["delta"], q["A"], q["B"], q["C"], D=q["D"],
                                   z=q["z"], delta_bias=q["delta_bias"])
        e = Errors(f"saved states after chunk {c}", TOL["f32"])
        e.add(host(states[:, c]), ref_h)
        e.report()
