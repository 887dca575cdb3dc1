"""GPU parity of the backward entry point (ss_scan_bwd) against the fp64 oracle's reverse-mode
gradients (oracle.scan_bwd, itself pinned by finite differences).

Comparison per gradient element, in the same form as the forward's: |gpu - oracle| <=
tol + tol * |oracle|, with tol = 1e-3 for float32 results (the recurrences and the sums over
channels and steps run in float32) and 2e-2 for results stored in bfloat16 (du, ddelta, dz with
bf16 io)."""
import numpy as np
import pytest

import oracle
from selective_state_space_36_amd import workloads as wl
from tests.helpers import dev, host

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


def check_grad(got, ref, tol, what):
    """Elementwise |got - ref| <= tol + tol * |ref|."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    bound = tol + tol * np.abs(ref)
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} outside atol=rtol={tol}; "
                             f"worst at {tuple(int(v) for v in i)}: got {got[i]!r} "
                             f"want {ref[i]!r}")


def run_bwd(p, *, gate=True, skip=True, h0=True, dh_last=True, softplus=True, seed=0, zoh=False):
    batch, L, D = p["u"].shape
    N = p["B"].shape[-1]
    rng = np.random.default_rng(seed)
    bf16 = p["u"].dtype == np.uint16
    g_out = rng.standard_normal((batch, L, D)).astype(np.float32)
    if bf16:
        g_out = wl.f32_to_bf16_bits(g_out)
    h0a = rng.standard_normal((batch, D, N)).astype(np.float32) if h0 else None
    dhl = rng.standard_normal((batch, D, N)).astype(np.float32) if dh_last else None
    z = p["z"] if gate else None
    Dk = p["D"] if skip else None
    print(f"  bwd case: shape={p['u'].shape} N={N} bf16={bf16} gate={gate} skip={skip} "
          f"h0={h0} dh_last={dh_last} softplus={softplus} zoh={zoh}", flush=True)
    g = ops().scan_bwd(dev(p["u"]), dev(p["delta"]), dev(p["A"]), dev(p["B"]), dev(p["C"]),
                       dev(g_out), D=dev(Dk), z=dev(z), delta_bias=dev(p["delta_bias"]),
                       delta_softplus=softplus, h0=dev(h0a), dh_last=dev(dhl), zoh_exact=zoh)
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"],
                          (wl_f64(g_out)), D=Dk, z=z, delta_bias=p["delta_bias"],
                          delta_softplus=softplus,
                          h0=None if h0a is None else h0a.astype(np.float64),
                          dh_last=None if dhl is None else dhl.astype(np.float64),
                          zoh_exact=zoh)
    io_tol = 2e-2 if bf16 else 1e-3
    for key in ("du", "ddelta", "dz"):
        if ref[key] is None or g[key] is None:
            assert (ref[key] is None) == (g[key] is None) or key == "dz"
            continue
        check_grad(host(g[key]), ref[key], io_tol, key)
    for key in ("dA", "dB", "dC", "dD", "ddelta_bias", "dh0"):
        check_grad(host(g[key]), ref[key], 1e-3, key)
    return g, ref


def wl_f64(x):
    """The exact value of an io-dtype array as float64."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


@pytest.mark.parametrize("gate,skip", [(False, True), (True, True), (True, False)])
def test_tiny_fp32_bwd(gate, skip):
    p = wl.make_prefill(wl.WORKLOADS[0])
    if gate:
        p["z"] = np.random.default_rng(3).standard_normal(p["u"].shape).astype(np.float32)
    run_bwd(p, gate=gate, skip=skip)


@pytest.mark.parametrize("batch,seqlen,d_inner", [(1, 1, 16), (2, 33, 17), (3, 300, 50),
                                                  (2, 256, 64), (2, 37, 32), (1, 100, 48)])
def test_bf16_ragged_bwd(batch, seqlen, d_inner):
    # d_inner a multiple of 16 takes the 16-byte tile path (gradients stored from LDS tiles),
    # with a partial last chunk when seqlen % 16 != 0; other widths the element path
    p = wl.make_prefill(wl.WORKLOADS[1], batch=batch, seqlen=seqlen, d_inner=d_inner, seed=41)
    run_bwd(p, seed=seqlen)


@pytest.mark.parametrize("seqlen", [45, 16])
def test_fp32_tile_path_bwd(seqlen):
    """fp32 io on the 16-byte tile path (four pieces per tile row), ragged and whole chunks."""
    p = wl.make_prefill(wl.WORKLOADS[0], batch=2, seqlen=seqlen, d_inner=32, seed=seqlen)
    run_bwd(p, gate=False, seed=seqlen)


@pytest.mark.parametrize("d_state", [1, 5, 16, 17, 24, 32, 33, 40, 64])
def test_state_sizes_bwd(d_state):
    p = wl.make_prefill(wl.WORKLOADS[0], batch=2, seqlen=70, d_inner=24, seed=d_state)
    rng = np.random.default_rng(d_state)
    p["B"] = rng.standard_normal((2, 70, d_state)).astype(np.float32)
    p["C"] = rng.standard_normal((2, 70, d_state)).astype(np.float32)
    p["A"] = np.ascontiguousarray(np.tile(-np.arange(1, d_state + 1, dtype=np.float32), (24, 1)))
    run_bwd(p, gate=False, seed=d_state)


def test_softplus_off_and_no_optional_inputs():
    p = wl.make_prefill(wl.WORKLOADS[0], batch=2, seqlen=50, d_inner=32, seed=6)
    p["delta"] = (np.abs(p["delta"]) * 0.1 + 0.01).astype(np.float32)
    p["delta_bias"] = None
    run_bwd(p, gate=False, skip=False, h0=False, dh_last=False, softplus=False)


# ------------------------------------------------------------------------------------------
# exact zero-order hold (SS_FLAG_ZOH_EXACT): gradients of (exp(dt A) - 1) / A * B u
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("gate,skip,softplus", [(False, True, True), (True, True, True),
                                                (True, False, False)])
def test_zoh_bwd_fp32(gate, skip, softplus):
    p = wl.make_prefill(wl.WORKLOADS[0], batch=2, seqlen=90, d_inner=32, seed=51)
    if gate:
        p["z"] = np.random.default_rng(4).standard_normal(p["u"].shape).astype(np.float32)
    if not softplus:  # dt used as given: positive, no bias
        p["delta"] = (np.abs(p["delta"]) * 0.1 + 0.01).astype(np.float32)
        p["delta_bias"] = None
    run_bwd(p, gate=gate, skip=skip, softplus=softplus, zoh=True, seed=51)


def test_zoh_bwd_mixed_A_covers_both_gain_forms():
    """A spread from 0 to -40 and dt from 1e-3 to ~1, so that |dt A log2 e| falls on both sides
    of the 1/8 switch between the series and the direct forms of the gain and of its derivative
    in A (A = 0 exactly in one column: the gain is dt, its derivative dt^2 / 2)."""
    rng = np.random.default_rng(61)
    p = wl.make_prefill(wl.WORKLOADS[0], batch=2, seqlen=70, d_inner=24, seed=61)
    A = -np.exp(rng.uniform(np.log(1e-3), np.log(40.0), size=(24, 16))).astype(np.float32)
    A[:, 3] = 0.0
    p["A"] = A
    p["delta_bias"] = rng.uniform(-7.0, 0.5, size=24).astype(np.float32)
    run_bwd(p, gate=False, zoh=True, seed=61)


@pytest.mark.parametrize("d_state", [1, 5])
def test_zoh_bwd_state_sizes(d_state):
    p = wl.make_prefill(wl.WORKLOADS[0], batch=2, seqlen=40, d_inner=20, seed=d_state)
    rng = np.random.default_rng(d_state)
    p["B"] = rng.standard_normal((2, 40, d_state)).astype(np.float32)
    p["C"] = rng.standard_normal((2, 40, d_state)).astype(np.float32)
    p["A"] = np.ascontiguousarray(np.tile(-np.arange(1, d_state + 1, dtype=np.float32), (20, 1)))
    run_bwd(p, gate=False, zoh=True, seed=d_state)


def test_zoh_bwd_bf16_and_repeatable():
    p = wl.make_prefill(wl.WORKLOADS[1], batch=2, seqlen=300, d_inner=48, seed=71)
    g1, _ = run_bwd(p, zoh=True, seed=71)
    g2, _ = run_bwd(p, zoh=True, seed=71)
    for key in ("du", "ddelta", "dz", "dh0", "dA", "dB", "dC", "dD", "ddelta_bias"):
        assert torch.equal(g1[key], g2[key]), key


@pytest.mark.parametrize("d_state", [32, 64])
def test_wide_state_bwd_bf16_with_given_states(d_state):
    """Wide states (two and four groups of 16 per lane) in bf16 with the gate, through both the
    recomputing backward and the one taking the states a forward saved, and repeatable."""
    p = wl.make_prefill(wl.WORKLOADS[1], batch=2, seqlen=200, d_inner=48, seed=d_state)
    rng = np.random.default_rng(d_state)
    mk = lambda: wl.f32_to_bf16_bits(rng.standard_normal((2, 200, d_state)).astype(np.float32))
    p["B"], p["C"] = mk(), mk()
    p["A"] = np.ascontiguousarray(np.tile(-np.arange(1, d_state + 1, dtype=np.float32), (48, 1)))
    g1, ref = run_bwd(p, seed=d_state)
    o = ops()
    args = [dev(p[k]) for k in ("u", "delta", "A", "B", "C")]
    kw = dict(D=dev(p["D"]), z=dev(p["z"]), delta_bias=dev(p["delta_bias"]))
    g_out = dev(wl.f32_to_bf16_bits(np.random.default_rng(d_state).standard_normal(
        p["u"].shape).astype(np.float32)))
    ws, states = o.bwd_workspace(2, 200, 48, d_state, torch.bfloat16)
    o.scan_fwd_states(*args, states=states, **kw)
    g_s = o.scan_bwd(*args, g_out, workspace=ws, states_given=True, **kw)
    g_r = o.scan_bwd(*args, g_out, **kw)
    g_r2 = o.scan_bwd(*args, g_out, **kw)
    torch.cuda.synchronize()
    for key in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0"):
        assert torch.equal(g_r[key], g_r2[key]), key
        tol = 2e-2 if key in ("du", "ddelta", "dz") else 1e-4
        check_grad(host(g_s[key]), host(g_r[key]), tol, key + " (given vs recomputed)")


@pytest.mark.parametrize("d_state", [24, 64])
def test_wide_state_zoh_bwd(d_state):
    p = wl.make_prefill(wl.WORKLOADS[0], batch=2, seqlen=40, d_inner=20, seed=d_state)
    rng = np.random.default_rng(d_state)
    p["B"] = rng.standard_normal((2, 40, d_state)).astype(np.float32)
    p["C"] = rng.standard_normal((2, 40, d_state)).astype(np.float32)
    p["A"] = (-np.exp(rng.uniform(np.log(1e-2), np.log(20.0), size=(20, d_state)))).astype(np.float32)
    run_bwd(p, gate=False, zoh=True, seed=d_state)


def test_zoh_bwd_rejects_given_states():
    o = ops()
    p = wl.make_prefill(wl.WORKLOADS[0], batch=1, seqlen=8, d_inner=16, seed=1)
    args = [dev(p[k]) for k in ("u", "delta", "A", "B", "C")]
    ws, states = o.bwd_workspace(1, 8, 16, 16, torch.float32)
    o.scan_fwd_states(*args, states=states)
    with pytest.raises(o.SSError) as e:
        o.scan_bwd(*args, dev(p["u"]), workspace=ws, states_given=True, zoh_exact=True)
    assert e.value.status == o.SS_ERR_UNSUPPORTED


def test_medium_bf16_bwd():
    """A 130M-shaped slice (batch 2, L 2048, d_inner 256) in bf16 with the gate."""
    p = wl.make_prefill(wl.WORKLOADS[1], batch=2, seqlen=2048, d_inner=256, seed=77)
    run_bwd(p, seed=77)


def test_bwd_repeatable():
    """Every gradient, the sums over channels and batch rows included, is bit-identical across
    calls (the partial sums are added in a fixed order)."""
    p = wl.make_prefill(wl.WORKLOADS[1], batch=2, seqlen=100, d_inner=48, seed=8)
    args = [dev(p[k]) for k in ("u", "delta", "A", "B", "C")]
    g_out = dev(wl.f32_to_bf16_bits(np.random.default_rng(8).standard_normal(
        p["u"].shape).astype(np.float32)))
    kw = dict(D=dev(p["D"]), z=dev(p["z"]), delta_bias=dev(p["delta_bias"]))
    g1 = ops().scan_bwd(*args, g_out, **kw)
    g2 = ops().scan_bwd(*args, g_out, **kw)
    torch.cuda.synchronize()
    for key in ("du", "ddelta", "dz", "dh0", "dA", "dB", "dC", "dD", "ddelta_bias"):
        assert torch.equal(g1[key], g2[key]), key


def test_bwd_full_size_bitwise_repeatable():
    """The 2.8B-shaped layer (320 channel blocks per batch row summed into dB and dC): two
    backward calls give the same bits for every gradient."""
    w = wl.WORKLOADS[2]
    p = wl.make_prefill(w)
    args = [dev(p[k]) for k in ("u", "delta", "A", "B", "C")]
    g_out = dev(wl.f32_to_bf16_bits(np.random.default_rng(9).standard_normal(
        p["u"].shape).astype(np.float32)))
    kw = dict(D=dev(p["D"]), z=dev(p["z"]), delta_bias=dev(p["delta_bias"]))
    g1 = ops().scan_bwd(*args, g_out, **kw)
    g2 = ops().scan_bwd(*args, g_out, **kw)
    torch.cuda.synchronize()
    for key in ("du", "ddelta", "dz", "dh0", "dA", "dB", "dC", "dD", "ddelta_bias"):
        assert torch.equal(g1[key], g2[key]), key


def test_invalid_bwd_arguments():
    o = ops()
    p = wl.make_prefill(wl.WORKLOADS[0], batch=1, seqlen=8, d_inner=16, seed=1)
    args = [dev(p[k]) for k in ("u", "delta", "A", "B", "C")]
    g_out = dev(p["u"])
    # d_state above 64
    B72 = torch.zeros((1, 8, 72), device="cuda")
    with pytest.raises(o.SSError) as e:
        o.scan_bwd(args[0], args[1], torch.zeros((16, 72), device="cuda"), B72, B72.clone(), g_out)
    assert e.value.status == o.SS_ERR_UNSUPPORTED
    # workspace too small
    with pytest.raises(o.SSError) as e:
        o.scan_bwd(*args, g_out, workspace=torch.empty(8, dtype=torch.uint8, device="cuda"))
    assert e.value.status == o.SS_ERR_INVALID_ARG
