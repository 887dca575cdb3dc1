"""GPU parity of the decode step with the fused front end (ss_state_update_conv) against the fp64
oracle's conv_step followed by its state_update, and the decode/prefill contract of the front
end: L such steps reproduce ss_scan_fwd_conv over the same L tokens given the same history."""
import dataclasses

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


def decode_inputs(io, *, steps, batch, d_inner, d_state, k, gate=True, seed=0):
    w = dataclasses.replace(wl.WORKLOADS[4], io_dtype=io, gate=gate, d_state=d_state)
    d = wl.make_decode(w, steps=steps, batch=batch, d_inner=d_inner, seed=seed)
    rng = np.random.default_rng(seed + 77)
    d["conv_w"] = (0.5 * rng.standard_normal((d_inner, k))).astype(np.float32)
    d["conv_b"] = (0.2 * rng.standard_normal(d_inner)).astype(np.float32)
    cs = rng.standard_normal((batch, k - 1, d_inner)).astype(np.float32)
    d["conv_state"] = wl.f32_to_bf16_bits(cs) if io == "bf16" else cs
    return d


def widen(a):
    """float32 or bf16 bits -> float64, exactly."""
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float64)


def run_steps(d, steps, *, gate=True, skip=True, bias=True, zoh=False):
    batch, d_inner, N = d["state"].shape
    k = d["conv_w"].shape[1]
    print(f"  decode conv case: batch={batch} d_inner={d_inner} N={N} k={k} "
          f"dtype={d['u'].dtype} gate={gate} skip={skip} bias={bias} zoh={zoh} steps={steps}",
          flush=True)
    st_gpu, cs_gpu = dev(d["state"]), dev(d["conv_state"])
    st_ref, cs_ref = d["state"].astype(np.float64), d["conv_state"].copy()
    cw, cb = dev(d["conv_w"]), dev(d["conv_b"]) if bias else None
    A, D, db = dev(d["A"]), dev(d["D"]) if skip else None, dev(d["delta_bias"])
    x_all, dl_all, B_all, C_all = (dev(d[n]) for n in ("u", "delta", "B", "C"))
    z_all = dev(d["z"]) if gate else None
    tol = TOL["bf16"] if d["u"].dtype == np.uint16 else TOL["f32"]
    for s in range(steps):
        out = ops().state_update_conv(
            st_gpu, cs_gpu, x_all[s], cw, cb, dl_all[s], A, B_all[s], C_all[s], D=D,
            z=None if z_all is None else z_all[s], delta_bias=db, zoh_exact=zoh)
        u, cs_ref = oracle.conv_step(cs_ref, d["u"][s], d["conv_w"],
                                     d["conv_b"] if bias else None)
        ref = oracle.state_update(st_ref, u, d["delta"][s], d["A"], d["B"][s], d["C"][s],
                                  D=d["D"] if skip else None, z=d["z"][s] if gate else None,
                                  delta_bias=d["delta_bias"], zoh_exact=zoh)
        check_close(host(out), ref, tol, f"decode conv step {s}")
        # The window shift moves stored values: bit-exact.
        np.testing.assert_array_equal(host(cs_gpu), widen(cs_ref), err_msg=f"conv_state step {s}")
    torch.cuda.synchronize()
    check_close(host(st_gpu), st_ref, 1e-4, "final state")


@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_conv_small(k, io):
    d = decode_inputs(io, steps=5, batch=3, d_inner=40, d_state=16, k=k, seed=k)
    run_steps(d, 5)


@pytest.mark.parametrize("d_state", [12, 20, 32, 64])
def test_decode_conv_state_sizes(d_state):
    d = decode_inputs("bf16", steps=4, batch=2, d_inner=33, d_state=d_state, k=4, seed=d_state)
    run_steps(d, 4)


@pytest.mark.parametrize("gate,skip,bias", [(False, False, False), (False, True, True),
                                            (True, False, False)])
def test_decode_conv_optional_inputs(gate, skip, bias):
    d = decode_inputs("f32", steps=3, batch=2, d_inner=24, d_state=16, k=4, gate=gate, seed=4)
    run_steps(d, 3, gate=gate, skip=skip, bias=bias)


def test_decode_conv_exact_hold():
    d = decode_inputs("bf16", steps=4, batch=2, d_inner=48, d_state=16, k=4, seed=8)
    run_steps(d, 4, zoh=True)


def test_decode_conv_matches_prefill_conv():
    """L decode steps with the front end reproduce one ss_scan_fwd_conv call over the same
    tokens whose x_prev is the initial window, and leave the same final state and window."""
    steps, batch, d_inner, k = 24, 2, 48, 4
    d = decode_inputs("f32", steps=steps, batch=batch, d_inner=d_inner, d_state=16, k=k, seed=3)
    o = ops()
    tr = lambda a: dev(np.ascontiguousarray(np.swapaxes(a, 0, 1)))  # (L, b, .) -> (b, L, .)
    pre, h_pre = o.scan_fwd_conv(tr(d["u"]), dev(d["conv_w"]), dev(d["conv_b"]), tr(d["delta"]),
                                 dev(d["A"]), tr(d["B"]), tr(d["C"]), D=dev(d["D"]),
                                 z=tr(d["z"]), delta_bias=dev(d["delta_bias"]),
                                 x_prev=dev(d["conv_state"]), h0=dev(d["state"]),
                                 return_last_state=True)
    st, cs = dev(d["state"]), dev(d["conv_state"])
    outs = []
    for s in range(steps):
        outs.append(o.state_update_conv(
            st, cs, dev(d["u"][s]), dev(d["conv_w"]), dev(d["conv_b"]), dev(d["delta"][s]),
            dev(d["A"]), dev(d["B"][s]), dev(d["C"][s]), D=dev(d["D"]), z=dev(d["z"][s]),
            delta_bias=dev(d["delta_bias"])))
    torch.cuda.synchronize()
    dec = np.stack([host(t) for t in outs], axis=1)
    check_close(dec, host(pre), 2e-5, "decode vs prefill out")
    check_close(host(st), host(h_pre), 2e-5, "decode vs prefill state")
    np.testing.assert_array_equal(host(cs), np.swapaxes(d["u"], 0, 1)[:, -(k - 1):, :])


def test_decode_conv_full_size():
    """The batch-128 decode layer (d_inner 5120, d_state 16, bf16) with the front end, three
    steps, every output checked."""
    w = wl.WORKLOADS[4]
    d = decode_inputs("bf16", steps=3, batch=w.batch, d_inner=w.d_inner, d_state=w.d_state, k=4,
                      seed=12)
    run_steps(d, 3)


def test_decode_conv_unsupported():
    o = ops()
    d = decode_inputs("f32", steps=1, batch=1, d_inner=16, d_state=16, k=4, seed=1)
    args = lambda dd, k: (dev(dd["state"]), dev(dd["conv_state"][:, :k - 1].copy()),
                          dev(dd["u"][0]), dev(dd["conv_w"][:, :k].copy()), None,
                          dev(dd["delta"][0]), dev(dd["A"]), dev(dd["B"][0]), dev(dd["C"][0]))
    for N in (8, 3):  # fewer than 16 lanes per channel, or no 4-wide state vectors
        dn = decode_inputs("f32", steps=1, batch=1, d_inner=16, d_state=N, k=4, seed=1)
        with pytest.raises(o.SSError) as e:
            o.state_update_conv(*args(dn, 4))
        assert e.value.status == o.SS_ERR_UNSUPPORTED
    w5 = torch.zeros((16, 5), device="cuda")
    cs5 = torch.zeros((1, 4, 16), device="cuda")
    with pytest.raises(o.SSError) as e:
        o.state_update_conv(dev(d["state"]), cs5, dev(d["u"][0]), w5, None, dev(d["delta"][0]),
                            dev(d["A"]), dev(d["B"][0]), dev(d["C"][0]))
    assert e.value.status == o.SS_ERR_UNSUPPORTED
