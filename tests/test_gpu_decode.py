"""GPU parity of the decode entry point (ss_state_update) against the fp64 oracle, and the
decode/prefill contract: L single-token steps reproduce the prefill outputs and final state."""
import numpy as np
import pytest

import oracle
from selective_state_space_36_amd import workloads as wl
from tests.helpers import TOL, check_close, dev, host

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


def _decode_steps(d, steps, rows=None, gate=True, skip=True):
    """Run `steps` GPU decode steps and the oracle's; compare every step's output (optionally on
    a row subset) and the final state."""
    batch, d_inner, N = d["state"].shape
    st_gpu = dev(d["state"])
    st_ref = d["state"].astype(np.float64)
    A, D, db = dev(d["A"]), dev(d["D"]) if skip else None, dev(d["delta_bias"])
    u_all, dl_all, B_all, C_all = (dev(d[k]) for k in ("u", "delta", "B", "C"))
    z_all = dev(d["z"]) if gate else None
    tol = TOL["bf16"] if d["u"].dtype == np.uint16 else TOL["f32"]
    for s in range(steps):
        out = ops().state_update(st_gpu, u_all[s], dl_all[s], A, B_all[s], C_all[s], D=D,
                                 z=None if z_all is None else z_all[s], delta_bias=db)
        ref = oracle.state_update(st_ref, d["u"][s], d["delta"][s], d["A"], d["B"][s], d["C"][s],
                                  D=d["D"] if skip else None, z=d["z"][s] if gate else None,
                                  delta_bias=d["delta_bias"], rows=rows)
        g = host(out).reshape(-1)
        if rows is not None:
            g = g[rows]
        check_close(g, ref.reshape(-1), tol, f"decode step {s}")
    torch.cuda.synchronize()
    gs = host(st_gpu).reshape(-1, N)
    rs = st_ref.reshape(-1, N)
    if rows is not None:
        gs, rs = gs[rows], rs[rows]
    check_close(gs, rs, 1e-4, "final state")


@pytest.mark.parametrize("d_state", [16, 1, 3, 8, 24, 64])
def test_decode_small(d_state):
    w = wl.WORKLOADS[4]
    d = wl.make_decode(w, steps=6, batch=3, d_inner=40)
    if d_state != 16:
        rng = np.random.default_rng(d_state)
        d["state"] = rng.standard_normal((3, 40, d_state)).astype(np.float32)
        d["A"] = np.ascontiguousarray(np.tile(-np.arange(1, d_state + 1, dtype=np.float32), (40, 1)))
        d["B"] = wl.f32_to_bf16_bits(rng.standard_normal((6, 3, d_state)).astype(np.float32))
        d["C"] = wl.f32_to_bf16_bits(rng.standard_normal((6, 3, d_state)).astype(np.float32))
    print(f"  decode small N={d_state}", flush=True)
    _decode_steps(d, 6)


def test_decode_unaligned_state_uses_generic_path():
    """A state buffer that is only 4-byte aligned takes the scalar path; same results."""
    w = wl.WORKLOADS[4]
    d = wl.make_decode(w, steps=3, batch=2, d_inner=24)
    flat = torch.empty(2 * 24 * 16 + 1, dtype=torch.float32, device="cuda")
    st = flat[1:].view(2, 24, 16)
    st.copy_(torch.from_numpy(d["state"]))
    st_ref = d["state"].astype(np.float64)
    for s in range(3):
        out = ops().state_update(st, dev(d["u"][s]), dev(d["delta"][s]), dev(d["A"]),
                                 dev(d["B"][s]), dev(d["C"][s]), D=dev(d["D"]), z=dev(d["z"][s]),
                                 delta_bias=dev(d["delta_bias"]))
        ref = oracle.state_update(st_ref, d["u"][s], d["delta"][s], d["A"], d["B"][s], d["C"][s],
                                  D=d["D"], z=d["z"][s], delta_bias=d["delta_bias"])
        check_close(host(out), ref, TOL["bf16"], f"step {s}")
    torch.cuda.synchronize()
    check_close(host(st), st_ref, 1e-4, "final state")


def test_decode_fp32_no_gate():
    rng = np.random.default_rng(5)
    batch, d_inner, N, steps = 4, 33, 16, 5
    d = dict(state=rng.standard_normal((batch, d_inner, N)).astype(np.float32),
             u=rng.standard_normal((steps, batch, d_inner)).astype(np.float32),
             delta=(0.5 * rng.standard_normal((steps, batch, d_inner))).astype(np.float32),
             z=None,
             B=rng.standard_normal((steps, batch, N)).astype(np.float32),
             C=rng.standard_normal((steps, batch, N)).astype(np.float32),
             A=-rng.uniform(0.5, 4, size=(d_inner, N)).astype(np.float32),
             D=rng.standard_normal(d_inner).astype(np.float32),
             delta_bias=rng.uniform(-4, -1, size=d_inner).astype(np.float32))
    _decode_steps(d, steps, gate=False)


def test_decode_reproduces_prefill():
    """L decode steps from h0 == one prefill of length L (outputs per step and final state)."""
    w = wl.WORKLOADS[1]
    p = wl.make_prefill(w, batch=2, seqlen=40, d_inner=64, seed=3)
    h0 = np.random.default_rng(9).standard_normal((2, 64, 16)).astype(np.float32)
    out, h_last = ops().scan_fwd(dev(p["u"]), dev(p["delta"]), dev(p["A"]), dev(p["B"]),
                                 dev(p["C"]), D=dev(p["D"]), z=dev(p["z"]),
                                 delta_bias=dev(p["delta_bias"]), h0=dev(h0),
                                 return_last_state=True)
    st = dev(h0)
    outs = []
    for t in range(40):
        sl = lambda k: dev(np.ascontiguousarray(p[k][:, t]))
        outs.append(ops().state_update(st, sl("u"), sl("delta"), dev(p["A"]), sl("B"), sl("C"),
                                       D=dev(p["D"]), z=sl("z"), delta_bias=dev(p["delta_bias"])))
    torch.cuda.synchronize()
    dec = host(torch.stack(outs, dim=1))
    check_close(dec, host(out), 1e-2, "decode vs prefill outputs")
    check_close(host(st), host(h_last), 1e-5, "decode vs prefill state")


def test_decode_invalid_arguments():
    o = ops()
    st = torch.zeros((2, 8, 16), device="cuda")
    u = torch.zeros((2, 8), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((2, 16), dtype=torch.bfloat16, device="cuda")
    A = -torch.ones((8, 16), device="cuda")
    with pytest.raises(o.SSError) as e:
        o.state_update(st, u, u.clone(), A, B, B.clone(), out=u)
    assert e.value.status == o.SS_ERR_INVALID_ARG


def test_decode_graph_replays_match_eager():
    """Decode steps captured into a HIP graph (as the benchmark's graph line does): each of
    several replays, with eager work and synchronisation between them, matches the same steps
    run eagerly from the same starting state, bit for bit."""
    w = wl.WORKLOADS[4]
    steps = 4
    d = wl.make_decode(w, steps=steps, batch=5, d_inner=96)
    A, D, db = dev(d["A"]), dev(d["D"]), dev(d["delta_bias"])
    u, dl, z, B, C = (dev(d[k]) for k in ("u", "delta", "z", "B", "C"))
    st0 = dev(d["state"])
    o = ops()

    def run(st, outs, stream):
        for s in range(steps):
            o.state_update(st, u[s], dl[s], A, B[s], C[s], D=D, z=z[s], delta_bias=db,
                           out=outs[s], stream=stream)

    st_e = st0.clone()
    outs_e = torch.empty((steps,) + u.shape[1:], dtype=u.dtype, device="cuda")
    run(st_e, outs_e, torch.cuda.current_stream())
    torch.cuda.synchronize()

    st_g = st0.clone()
    outs_g = torch.empty_like(outs_e)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        run(st_g, outs_g, cap)  # warm-up outside the capture
        cap.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            run(st_g, outs_g, cap)
    torch.cuda.synchronize()
    for rep in range(3):
        st_g.copy_(st0)
        outs_g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs_g, outs_e), f"replay {rep}: outputs differ from eager"
        assert torch.equal(st_g, st_e), f"replay {rep}: state differs from eager"
