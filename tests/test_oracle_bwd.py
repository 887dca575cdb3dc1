"""Pins of the oracle's gradients (oracle_scan_bwd): central finite differences of the forward
oracle on tiny float32 inputs, and a closed form for the decay-free linear case.  The forward
oracle is pinned on its own (test_oracle_pins.py), so these check the reverse-mode derivation
against the function it differentiates."""
import numpy as np
import pytest

import oracle

H = 2.0 ** -14  # finite-difference step


def _case(rng, batch=2, L=6, D=3, N=4, gate=True, skip=True, bias=True):
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    c = dict(u=f(batch, L, D), delta=(0.5 * f(batch, L, D)).astype(np.float32),
             A=(-np.exp(rng.uniform(-1, 1, (D, N)))).astype(np.float32), B=f(batch, L, N),
             C=f(batch, L, N), D=f(D) if skip else None, z=f(batch, L, D) if gate else None,
             delta_bias=(0.3 * f(D)).astype(np.float32) if bias else None,
             h0=rng.standard_normal((batch, D, N)))
    w_out = rng.standard_normal((batch, L, D))
    w_h = rng.standard_normal((batch, D, N))
    return c, w_out, w_h


def _loss(c, w_out, w_h, softplus=True, zoh=False):
    out, h = oracle.scan_fwd(c["u"], c["delta"], c["A"], c["B"], c["C"], D=c["D"], z=c["z"],
                             delta_bias=c["delta_bias"], delta_softplus=softplus, h0=c["h0"],
                             zoh_exact=zoh)
    return float(np.sum(w_out * out) + np.sum(w_h * h))


def _fd(c, key, w_out, w_h, softplus=True, zoh=False):
    """Central difference of the loss in every element of c[key].  The perturbed values are
    rounded to the input's dtype, so the difference quotient divides by the step actually taken
    (it differs from 2H only where x +- H crosses a power of two)."""
    base = c[key]
    grad = np.zeros(base.shape)
    for idx in np.ndindex(base.shape):
        vals, xs = [], []
        for sgn in (1, -1):
            pert = base.copy()
            pert[idx] = pert[idx] + sgn * H
            xs.append(float(pert[idx]))
            c2 = dict(c)
            c2[key] = pert
            vals.append(_loss(c2, w_out, w_h, softplus, zoh))
        grad[idx] = (vals[0] - vals[1]) / (xs[0] - xs[1])
    return grad


KEYS = [("u", "du"), ("delta", "ddelta"), ("z", "dz"), ("A", "dA"), ("B", "dB"), ("C", "dC"),
        ("D", "dD"), ("delta_bias", "ddelta_bias"), ("h0", "dh0")]


@pytest.mark.parametrize("softplus", [True, False])
def test_gradients_match_finite_differences(softplus):
    rng = np.random.default_rng(1 + softplus)
    c, w_out, w_h = _case(rng)
    if not softplus:  # keep dt positive without softplus
        c["delta"] = np.abs(c["delta"]) + np.float32(0.1)
    g = oracle.scan_bwd(c["u"], c["delta"], c["A"], c["B"], c["C"], w_out, D=c["D"], z=c["z"],
                        delta_bias=c["delta_bias"], delta_softplus=softplus, h0=c["h0"],
                        dh_last=w_h)
    for key, gk in KEYS:
        fd = _fd(c, key, w_out, w_h, softplus)
        np.testing.assert_allclose(g[gk], fd, rtol=1e-6, atol=1e-7, err_msg=gk)


@pytest.mark.parametrize("softplus", [True, False])
def test_exact_zoh_gradients_match_finite_differences(softplus):
    """The exact zero-order-hold input term (exp(dt a) - 1) / a * B: its derivatives in dt and a
    enter ddelta, du, dB and dA; finite differences of the exact-ZOH forward oracle pin them."""
    rng = np.random.default_rng(11 + softplus)
    c, w_out, w_h = _case(rng)
    if not softplus:
        c["delta"] = np.abs(c["delta"]) + np.float32(0.1)
    g = oracle.scan_bwd(c["u"], c["delta"], c["A"], c["B"], c["C"], w_out, D=c["D"], z=c["z"],
                        delta_bias=c["delta_bias"], delta_softplus=softplus, h0=c["h0"],
                        dh_last=w_h, zoh_exact=True)
    for key, gk in KEYS:
        fd = _fd(c, key, w_out, w_h, softplus, zoh=True)
        np.testing.assert_allclose(g[gk], fd, rtol=1e-6, atol=1e-7, err_msg=gk)


def test_exact_zoh_gradient_at_zero_decay():
    """A column of A equal to 0: the exact-ZOH gain is dt there, and its derivative in a is
    dt^2 / 2 (the limit); a one-sided finite difference from a = 0 into a < 0 pins it."""
    rng = np.random.default_rng(13)
    c, w_out, w_h = _case(rng, gate=False)
    c["A"][:, 1] = 0.0
    g = oracle.scan_bwd(c["u"], c["delta"], c["A"], c["B"], c["C"], w_out, D=c["D"],
                        delta_bias=c["delta_bias"], h0=c["h0"], dh_last=w_h, zoh_exact=True)
    step = 2.0 ** -12
    for d in range(c["A"].shape[0]):
        vals = []
        for k in (0, 1, 2):
            c2 = dict(c)
            c2["A"] = c["A"].copy()
            c2["A"][d, 1] = -k * step
            vals.append(_loss(c2, w_out, w_h, zoh=True))
        # second-order one-sided difference: f'(0) ~ (3 f(0) - 4 f(-h) + f(-2h)) / (2h)
        fd = (3 * vals[0] - 4 * vals[1] + vals[2]) / (2 * step)
        np.testing.assert_allclose(g["dA"][d, 1], fd, rtol=1e-5, atol=1e-6)


def test_summed_gradients_do_not_depend_on_thread_count():
    """The sums over rows (dA, dB, dC, dD, ddelta_bias) run in per-thread partials; any thread
    count gives the same values to rounding, and one count gives the same bits every time."""
    rng = np.random.default_rng(17)
    c, w_out, w_h = _case(rng, batch=3, L=20, D=13, N=5)
    run = lambda nt: oracle.scan_bwd(c["u"], c["delta"], c["A"], c["B"], c["C"], w_out, D=c["D"],
                                     z=c["z"], delta_bias=c["delta_bias"], h0=c["h0"],
                                     dh_last=w_h, nthreads=nt)
    g1, g4, g4b = run(1), run(4), run(4)
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0"):
        np.testing.assert_allclose(g4[k], g1[k], rtol=1e-12, atol=1e-14, err_msg=k)
        np.testing.assert_array_equal(g4[k], g4b[k], err_msg=k)


def test_without_gate_skip_bias_or_h0():
    rng = np.random.default_rng(7)
    c, w_out, w_h = _case(rng, gate=False, skip=False, bias=False)
    c["h0"] = None
    g = oracle.scan_bwd(c["u"], c["delta"], c["A"], c["B"], c["C"], w_out, delta_bias=None,
                        dh_last=None)
    assert g["dz"] is None
    for key, gk in [("u", "du"), ("delta", "ddelta"), ("A", "dA"), ("B", "dB"), ("C", "dC")]:
        fd = _fd(c, key, w_out, np.zeros_like(w_h))
        np.testing.assert_allclose(g[gk], fd, rtol=1e-6, atol=1e-7, err_msg=gk)
    # the gradient at D = 0 is sum_t dout * u, and dh0 is what reaches the zero initial state
    np.testing.assert_allclose(g["dD"], np.einsum("btd,btd->d", w_out, c["u"]), rtol=1e-12)


def test_decay_free_linear_closed_form():
    """A = 0, softplus off, no gate, D = 0: out_t = sum_n C_t[n] sum_{s<=t} dt_s B_s[n] u_s, so
    d(sum_t w_t out_t)/du_s = dt_s sum_n B_s[n] sum_{t>=s} w_t C_t[n] (a reversed cumulative sum)
    and d/dC_t[n] = w_t h_t[n] summed over channels."""
    rng = np.random.default_rng(9)
    batch, L, D, N = 2, 11, 3, 5
    u = rng.standard_normal((batch, L, D)).astype(np.float32)
    dt = rng.uniform(0.1, 1.0, (batch, L, D)).astype(np.float32)
    A = np.zeros((D, N), np.float32)
    B = rng.standard_normal((batch, L, N)).astype(np.float32)
    C = rng.standard_normal((batch, L, N)).astype(np.float32)
    w = rng.standard_normal((batch, L, D))
    g = oracle.scan_bwd(u, dt, A, B, C, w, delta_softplus=False)
    u64, dt64, B64, C64 = (x.astype(np.float64) for x in (u, dt, B, C))
    # sum_{t>=s} w_t[b,d] C_t[b,n]  -> (batch, L, D, N)
    wc = np.einsum("btd,btn->btdn", w, C64)[:, ::-1].cumsum(axis=1)[:, ::-1]
    du = dt64 * np.einsum("bsn,bsdn->bsd", B64, wc)
    np.testing.assert_allclose(g["du"], du, rtol=1e-12, atol=1e-12)
    h = np.cumsum(np.einsum("bsd,bsn->bsdn", dt64 * u64, B64), axis=1)
    np.testing.assert_allclose(g["dC"], np.einsum("btd,btdn->btn", w, h), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dB"], np.einsum("bsdn,bsd->bsn", wc, dt64 * u64), rtol=1e-12,
                               atol=1e-12)


def test_empty_sequence_passes_dh_last_to_dh0():
    rng = np.random.default_rng(3)
    c, _, w_h = _case(rng, L=0)
    g = oracle.scan_bwd(c["u"], c["delta"], c["A"], c["B"], c["C"], np.zeros((2, 0, 3)),
                        D=c["D"], h0=c["h0"], dh_last=w_h)
    np.testing.assert_array_equal(g["dh0"], w_h)
    assert not g["dA"].any() and not g["dD"].any()
