"""GPU parity of the fused front end (ss_scan_fwd_conv: u = silu(causal depthwise conv of x), then
the scan) against the fp64 oracle's conv_silu followed by its scan, on the same bytes."""
import numpy as np
import pytest

import oracle
from selective_state_space_36_amd import workloads as wl
from tests.helpers import TOL, check_close, check_every_row, dev, host

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


def conv_params(rng, d_inner, k, io, prev_batch=None):
    w = (0.5 * rng.standard_normal((d_inner, k))).astype(np.float32)
    b = (0.2 * rng.standard_normal(d_inner)).astype(np.float32)
    xp = None
    if prev_batch is not None and k > 1:
        xp = rng.standard_normal((prev_batch, k - 1, d_inner)).astype(np.float32)
        if io == "bf16":
            xp = wl.f32_to_bf16_bits(xp)
    return w, b, xp


def run_conv(p, w, b, xp, *, gate=True, skip=True, h0=None, nseg=None, zoh=False, rows=None):
    """p["u"] plays the block's x.  Returns (gpu_out, gpu_h, ref_out, ref_h)."""
    z = p["z"] if gate else None
    D = p["D"] if skip else None
    print(f"  conv case: shape={p['u'].shape} N={p['B'].shape[-1]} k={w.shape[1]} "
          f"dtype={p['u'].dtype} prev={xp is not None} gate={gate} nseg={nseg} zoh={zoh}",
          flush=True)
    out, h_last = ops().scan_fwd_conv(
        dev(p["u"]), dev(w), dev(b), dev(p["delta"]), dev(p["A"]), dev(p["B"]), dev(p["C"]),
        D=dev(D), z=dev(z), delta_bias=dev(p["delta_bias"]), x_prev=dev(xp),
        h0=None if h0 is None else dev(h0), return_last_state=True, nseg=nseg, zoh_exact=zoh)
    torch.cuda.synchronize()
    u = oracle.conv_silu(p["u"], w, b, x_prev=xp)
    ref_out, ref_h = oracle.scan_fwd(u, p["delta"], p["A"], p["B"], p["C"], D=D, z=z,
                                     delta_bias=p["delta_bias"], zoh_exact=zoh, rows=rows,
                                     h0=None if h0 is None else h0.astype(np.float64))
    return host(out), host(h_last), ref_out, ref_h


@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("prev", [False, True])
def test_tiny_fp32_conv(k, prev):
    p = wl.make_prefill(wl.WORKLOADS[0], batch=2, seqlen=70, d_inner=24, seed=k)
    w, b, xp = conv_params(np.random.default_rng(k), 24, k, "f32", 2 if prev else None)
    g, gh, r, rh = run_conv(p, w, b, xp, gate=False)
    check_close(g, r, TOL["f32"], "out")
    check_close(gh, rh, TOL["f32"], "h_last")


@pytest.mark.parametrize("batch,seqlen,d_inner", [(1, 1, 16), (2, 3, 17), (2, 33, 50),
                                                  (3, 300, 64)])
def test_bf16_ragged_conv(batch, seqlen, d_inner):
    p = wl.make_prefill(wl.WORKLOADS[1], batch=batch, seqlen=seqlen, d_inner=d_inner, seed=13)
    w, b, xp = conv_params(np.random.default_rng(seqlen), d_inner, 4, "bf16", batch)
    g, gh, r, rh = run_conv(p, w, b, xp)
    check_close(g, r, TOL["bf16"], "out")
    check_close(gh, rh, TOL["f32"], "h_last")


@pytest.mark.parametrize("nseg", [2, 7])
def test_time_split_conv(nseg):
    """Segments that start mid-sequence take their first taps from x before the segment."""
    p = wl.make_prefill(wl.WORKLOADS[0], batch=1, seqlen=1000, d_inner=32, seed=21)
    w, b, xp = conv_params(np.random.default_rng(21), 32, 4, "f32", 1)
    h0 = np.random.default_rng(22).standard_normal((1, 32, 16)).astype(np.float32)
    g, gh, r, rh = run_conv(p, w, b, xp, gate=False, h0=h0, nseg=nseg)
    check_close(g, r, TOL["f32"], "out")
    check_close(gh, rh, TOL["f32"], "h_last")


@pytest.mark.parametrize("d_state", [1, 17, 64])
def test_state_sizes_conv(d_state):
    p = wl.make_prefill(wl.WORKLOADS[0], batch=2, seqlen=50, d_inner=20, seed=d_state)
    rng = np.random.default_rng(d_state)
    p["B"] = rng.standard_normal((2, 50, d_state)).astype(np.float32)
    p["C"] = rng.standard_normal((2, 50, d_state)).astype(np.float32)
    p["A"] = np.ascontiguousarray(np.tile(-np.arange(1, d_state + 1, dtype=np.float32), (20, 1)))
    w, b, xp = conv_params(rng, 20, 3, "f32", 2)
    g, gh, r, rh = run_conv(p, w, b, xp, gate=False)
    check_close(g, r, TOL["f32"], "out")
    check_close(gh, rh, TOL["f32"], "h_last")


def test_conv_with_exact_hold():
    p = wl.make_prefill(wl.WORKLOADS[1], batch=2, seqlen=100, d_inner=48, seed=5)
    w, b, xp = conv_params(np.random.default_rng(5), 48, 4, "bf16", 2)
    g, gh, r, rh = run_conv(p, w, b, xp, zoh=True)
    check_close(g, r, TOL["bf16"], "out")
    check_close(gh, rh, TOL["f32"], "h_last")


def test_split_call_resumes_with_history():
    """Two calls, the second given the first's final state and its last k-1 inputs as x_prev,
    reproduce one call over the whole sequence."""
    p = wl.make_prefill(wl.WORKLOADS[0], batch=2, seqlen=96, d_inner=32, seed=9)
    w, b, _ = conv_params(np.random.default_rng(9), 32, 4, "f32")
    o = ops()
    whole, hw = o.scan_fwd_conv(dev(p["u"]), dev(w), dev(b), dev(p["delta"]), dev(p["A"]),
                                dev(p["B"]), dev(p["C"]), D=dev(p["D"]),
                                delta_bias=dev(p["delta_bias"]), return_last_state=True)
    cut = 37
    first, sl2 = slice(0, cut), slice(cut, None)
    part = lambda k, sl: dev(np.ascontiguousarray(p[k][:, sl]))
    o1, h1 = o.scan_fwd_conv(part("u", first), dev(w), dev(b), part("delta", first), dev(p["A"]),
                             part("B", first), part("C", first), D=dev(p["D"]),
                             delta_bias=dev(p["delta_bias"]), return_last_state=True)
    xp = dev(np.ascontiguousarray(p["u"][:, cut - 3:cut]))
    o2, h2 = o.scan_fwd_conv(part("u", sl2), dev(w), dev(b), part("delta", sl2), dev(p["A"]),
                             part("B", sl2), part("C", sl2), D=dev(p["D"]),
                             delta_bias=dev(p["delta_bias"]), x_prev=xp, h0=h1,
                             return_last_state=True)
    torch.cuda.synchronize()
    check_close(host(torch.cat([o1, o2], dim=1)), host(whole), 1e-5, "split out")
    check_close(host(h2), host(hw), 1e-5, "split h_last")


def test_invalid_conv_arguments():
    o = ops()
    p = wl.make_prefill(wl.WORKLOADS[0], batch=1, seqlen=8, d_inner=16, seed=1)
    w5 = torch.zeros((16, 5), device="cuda")
    with pytest.raises(o.SSError) as e:
        o.scan_fwd_conv(dev(p["u"]), w5, None, dev(p["delta"]), dev(p["A"]), dev(p["B"]),
                        dev(p["C"]))
    assert e.value.status == o.SS_ERR_UNSUPPORTED


def test_full_size_conv_every_row():
    """The 2.8B-shaped layer (batch 4, L 4096, d_inner 5120) through the front end, in the
    launch configuration the benchmark uses, every row checked: the oracle runs the front end
    and the scan on each block of channels (channels are independent)."""
    w_ = wl.WORKLOADS[2]
    p = wl.make_prefill(w_)
    w, b, xp = conv_params(np.random.default_rng(2), w_.d_inner, 4, "bf16", w_.batch)
    print("  conv full size: GPU", flush=True)
    out, h_last = ops().scan_fwd_conv(
        dev(p["u"]), dev(w), dev(b), dev(p["delta"]), dev(p["A"]), dev(p["B"]), dev(p["C"]),
        D=dev(p["D"]), z=dev(p["z"]), delta_bias=dev(p["delta_bias"]), x_prev=dev(xp),
        return_last_state=True)
    torch.cuda.synchronize()

    def reference(bi, d0, d1):
        blk = lambda a: np.ascontiguousarray(a[bi:bi + 1, :, d0:d1])
        u = oracle.conv_silu(blk(p["u"]), w[d0:d1], b[d0:d1], x_prev=blk(xp))
        r, rh = oracle.scan_fwd(u, blk(p["delta"]), p["A"][d0:d1],
                                np.ascontiguousarray(p["B"][bi:bi + 1]),
                                np.ascontiguousarray(p["C"][bi:bi + 1]), D=p["D"][d0:d1],
                                z=blk(p["z"]), delta_bias=p["delta_bias"][d0:d1])
        return r[0].T, rh[0]

    check_every_row(out, h_last, reference, "conv front end, 2.8B layer", out_tol=TOL["bf16"],
                    h_tol=TOL["f32"])
