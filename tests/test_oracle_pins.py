"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each test checks the oracle against something other than itself: a hand-worked example, a
closed form, a library routine (numpy.convolve, numpy.cumsum, scipy's expit, numpy's
logaddexp), brute force on tiny inputs, or a structural invariant.  Together they are chosen so
that a plausible slip in the oracle -- a dropped term, a wrong sign or index, a transposed
operand, y taken from h_{t-1} instead of h_t, the bias added after softplus, D inside or outside
the gate -- fails at least one of them.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit

import oracle
from oracle import numpy_twin

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.txt")
LN2 = np.log(2.0)


def softplus(s):
    return np.logaddexp(0.0, s)


def f64(x):
    return np.asarray(x, dtype=np.float64)


def rand_case(rng, batch=2, L=9, d_inner=3, N=4, bf16=False):
    def arr(*shape, scale=1.0):
        x = (rng.standard_normal(shape) * scale).astype(np.float32)
        if bf16:
            b = x.view(np.uint32)
            return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
        return x
    return dict(
        u=arr(batch, L, d_inner), delta=arr(batch, L, d_inner, scale=0.7),
        z=arr(batch, L, d_inner), B=arr(batch, L, N), C=arr(batch, L, N),
        A=-rng.uniform(0.2, 3.0, size=(d_inner, N)).astype(np.float32),
        D=rng.standard_normal(d_inner).astype(np.float32),
        delta_bias=rng.uniform(-3, 0, size=d_inner).astype(np.float32),
        h0=rng.standard_normal((batch, d_inner, N)))


def widen(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        import torch
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    return x.astype(np.float64)


# ------------------------------------------------------------------------------------------
# Hand-worked examples (golden fixtures)
# ------------------------------------------------------------------------------------------
def _parse_golden():
    cases, cur = {}, None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, val = line.partition(":")
        key, val = key.strip(), val.strip()
        if key == "case":
            cur = cases.setdefault(val, {})
        else:
            cur[key] = val.split()
    return cases


def _exact(tok):
    if tok.endswith("*ln2"):
        return float(Fraction(tok[:-4])) * LN2
    return float(Fraction(tok))


@pytest.mark.parametrize("zoh", [False, True])
@pytest.mark.parametrize("name", ["gated_rnn", "sum_and_reset"])
def test_golden_worked_examples(name, zoh):
    c = _parse_golden()[name]
    N = int(c["d_state"][0])
    L = len(c["u"])
    f = lambda k: np.array([float(Fraction(v)) for v in c[k]], dtype=np.float32)
    u = f("u").reshape(1, L, 1)
    delta = f("delta").reshape(1, L, 1)
    A = f("A").reshape(1, N)
    B = f("B").reshape(1, L, N)
    C = f("C").reshape(1, L, N)
    D = f("D") if "D" in c else None
    h0 = f("h0").astype(np.float64).reshape(1, 1, N)
    out, h_last = oracle.scan_fwd(u, delta, A, B, C, D=D, delta_softplus=bool(int(c["delta_softplus"][0])),
                                  h0=h0, zoh_exact=zoh)
    tag = "zoh_exact" if zoh else "first_order"
    want = np.array([_exact(t) for t in c["expect_" + tag]])
    want_h = np.array([_exact(t) for t in c["expect_" + tag + "_h_last"]])
    np.testing.assert_allclose(out[0, :, 0], want, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(h_last[0, 0], want_h, rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------------------------------------
# P-a: dt == 0 -> the input never reaches the state; y = D u (gated), h stays h0
# ------------------------------------------------------------------------------------------
def test_zero_step_gives_skip_only_exactly():
    rng = np.random.default_rng(1)
    c = rand_case(rng)
    zero = np.zeros_like(c["delta"])
    out, h_last = oracle.scan_fwd(c["u"], zero, c["A"], c["B"], c["C"], D=c["D"],
                                  delta_softplus=False)
    want = c["D"].astype(np.float64)[None, None, :] * c["u"].astype(np.float64)
    assert np.array_equal(out, want)                    # bit-exact: 0 + D*u in fp64
    assert np.array_equal(h_last, np.zeros_like(h_last))
    # with the gate: D*u*silu(z), silu from scipy's logistic
    out_g, _ = oracle.scan_fwd(c["u"], zero, c["A"], c["B"], c["C"], D=c["D"], z=c["z"],
                               delta_softplus=False)
    zz = c["z"].astype(np.float64)
    np.testing.assert_allclose(out_g, want * zz * expit(zz), rtol=1e-14, atol=0)
    # with an initial state: h_t == h0 for all t, y_t = C_t . h0 + D u_t
    out_h, h_last_h = oracle.scan_fwd(c["u"], zero, c["A"], c["B"], c["C"], D=c["D"],
                                      delta_softplus=False, h0=c["h0"])
    want_h = np.einsum("btn,bdn->btd", c["C"].astype(np.float64), c["h0"]) + want
    np.testing.assert_allclose(out_h, want_h, rtol=1e-14, atol=1e-14)
    assert np.array_equal(h_last_h, c["h0"])


# ------------------------------------------------------------------------------------------
# P-b: time-invariant case == causal convolution with K_k = sum_n C_n exp(dt A_n)^k dt B_n
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("with_h0", [False, True])
def test_time_invariant_equals_convolution(with_h0):
    rng = np.random.default_rng(2)
    batch, L, d_inner, N = 2, 40, 3, 5
    u = rng.standard_normal((batch, L, d_inner)).astype(np.float32)
    raw = rng.uniform(-2, 1, size=(batch, 1, d_inner)).astype(np.float32)
    delta = np.repeat(raw, L, axis=1)
    Bc = rng.standard_normal((batch, 1, N)).astype(np.float32)
    Cc = rng.standard_normal((batch, 1, N)).astype(np.float32)
    B, C = np.repeat(Bc, L, axis=1), np.repeat(Cc, L, axis=1)
    A = -rng.uniform(0.05, 1.5, size=(d_inner, N)).astype(np.float32)
    D = rng.standard_normal(d_inner).astype(np.float32)
    h0 = rng.standard_normal((batch, d_inner, N)) if with_h0 else None
    out, _ = oracle.scan_fwd(u, delta, A, B, C, D=D, h0=h0)
    k = np.arange(L)
    for b in range(batch):
        for d in range(d_inner):
            dt = softplus(float(raw[b, 0, d]))
            abar = np.exp(dt * A[d].astype(np.float64))                    # (N,)
            Bn, Cn = Bc[b, 0].astype(np.float64), Cc[b, 0].astype(np.float64)
            K = (Cn[None, :] * np.power(abar[None, :], k[:, None]) * dt * Bn[None, :]).sum(1)
            want = (np.convolve(u[b, :, d].astype(np.float64), K)[:L]
                    + float(D[d]) * u[b, :, d].astype(np.float64))
            if with_h0:
                want += (Cn[None, :] * np.power(abar[None, :], k[:, None] + 1)
                         * h0[b, d][None, :]).sum(1)
            np.testing.assert_allclose(out[b, :, d], want, rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------------------------------------
# P-c: A == 0 -> the state is a prefix sum of dt_s B_s u_s
# ------------------------------------------------------------------------------------------
def test_no_decay_is_prefix_sum():
    rng = np.random.default_rng(3)
    c = rand_case(rng, L=30)
    A = np.zeros_like(c["A"])
    out, h_last = oracle.scan_fwd(c["u"], c["delta"], A, c["B"], c["C"], D=c["D"],
                                  delta_bias=c["delta_bias"], h0=c["h0"])
    dt = softplus(c["delta"].astype(np.float64) + c["delta_bias"].astype(np.float64))
    inj = dt[..., None] * c["B"].astype(np.float64)[:, :, None, :] * \
        c["u"].astype(np.float64)[..., None]                               # (b, t, d, n)
    h = c["h0"][:, None] + np.cumsum(inj, axis=1)
    want = np.einsum("btdn,btn->btd", h, c["C"].astype(np.float64)) + f64(c["D"]) * f64(c["u"])
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h_last, h[:, -1], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------------------
# P-d: B == 0 with h0 != 0 -> pure decay h_t = exp(A * sum_{s<=t} dt_s) h0
# ------------------------------------------------------------------------------------------
def test_pure_decay_of_initial_state():
    rng = np.random.default_rng(4)
    c = rand_case(rng, L=50)
    B = np.zeros_like(c["B"])
    out, h_last = oracle.scan_fwd(c["u"], c["delta"], c["A"], B, c["C"], D=c["D"],
                                  delta_bias=c["delta_bias"], h0=c["h0"])
    dt = softplus(c["delta"].astype(np.float64) + c["delta_bias"].astype(np.float64))
    S = np.cumsum(dt, axis=1)                                              # (b, t, d)
    h = np.exp(S[..., None] * c["A"].astype(np.float64)[None, None]) * c["h0"][:, None]
    want = np.einsum("btdn,btn->btd", h, c["C"].astype(np.float64)) + f64(c["D"]) * f64(c["u"])
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(h_last, h[:, -1], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------------------------------
# P-e: N = 1, A = -1, B = 1 is a gated RNN (reading guide, section on the selection mechanism)
# ------------------------------------------------------------------------------------------
def test_gated_rnn_special_case():
    rng = np.random.default_rng(5)
    L = 64
    s = rng.uniform(-6, 6, size=(1, L, 1)).astype(np.float32)
    u = rng.standard_normal((1, L, 1)).astype(np.float32)
    one = np.ones((1, L, 1), np.float32)
    A = -np.ones((1, 1), np.float32)
    out_zoh, _ = oracle.scan_fwd(u, s, A, one, one, zoh_exact=True)
    out_fo, _ = oracle.scan_fwd(u, s, A, one, one, zoh_exact=False)
    g = expit(s.astype(np.float64)[0, :, 0])
    x = u.astype(np.float64)[0, :, 0]
    h1 = h2 = 0.0
    for t in range(L):
        h1 = (1 - g[t]) * h1 + g[t] * x[t]                  # textbook gated update
        h2 = expit(-float(s[0, t, 0])) * h2 + softplus(float(s[0, t, 0])) * x[t]
        assert abs(out_zoh[0, t, 0] - h1) <= 1e-13 * (1 + abs(h1))
        assert abs(out_fo[0, t, 0] - h2) <= 1e-13 * (1 + abs(h2))


# ------------------------------------------------------------------------------------------
# P-f: unrolled (materialised) form, brute force on tiny inputs
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("zoh", [False, True])
def test_unrolled_brute_force(zoh):
    rng = np.random.default_rng(6)
    c = rand_case(rng, batch=2, L=7, d_inner=2, N=3)
    out, h_last = oracle.scan_fwd(c["u"], c["delta"], c["A"], c["B"], c["C"], D=c["D"],
                                  z=c["z"], delta_bias=c["delta_bias"], h0=c["h0"],
                                  zoh_exact=zoh)
    u, Bm, Cm, z = (x.astype(np.float64) for x in (c["u"], c["B"], c["C"], c["z"]))
    A = c["A"].astype(np.float64)
    dt = softplus(c["delta"].astype(np.float64) + c["delta_bias"].astype(np.float64))
    batch, L, d_inner = u.shape
    N = A.shape[1]
    for b in range(batch):
        for d in range(d_inner):
            for t in range(L):
                y = 0.0
                for n in range(N):
                    a = A[d, n]
                    for s_ in range(t + 1):
                        decay = np.exp(a * dt[b, s_ + 1:t + 1, d].sum())
                        fac = np.expm1(dt[b, s_, d] * a) / a if zoh else dt[b, s_, d]
                        y += Cm[b, t, n] * decay * fac * Bm[b, s_, n] * u[b, s_, d]
                    y += Cm[b, t, n] * np.exp(a * dt[b, :t + 1, d].sum()) * c["h0"][b, d, n]
                y += float(c["D"][d]) * u[b, t, d]
                y *= z[b, t, d] * expit(z[b, t, d])
                assert abs(out[b, t, d] - y) <= 1e-12 * (1 + abs(y)), (b, t, d)


# ------------------------------------------------------------------------------------------
# P-g: the blockwise associative decomposition equals the sequential recurrence
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("chunk", [1, 3, 16, 64, 100])
def test_chunked_equals_sequential(chunk):
    rng = np.random.default_rng(7)
    c = rand_case(rng, batch=2, L=100, d_inner=3, N=4)
    kw = dict(D=c["D"], z=c["z"], delta_bias=c["delta_bias"], h0=c["h0"])
    for zoh in (False, True):
        seq, h_seq = oracle.scan_fwd(c["u"], c["delta"], c["A"], c["B"], c["C"], zoh_exact=zoh, **kw)
        chk, h_chk = oracle.scan_fwd_chunked(c["u"], c["delta"], c["A"], c["B"], c["C"], chunk,
                                             zoh_exact=zoh, **kw)
        np.testing.assert_allclose(chk, seq, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(h_chk, h_seq, rtol=1e-12, atol=1e-12)


def test_combine_operator_is_associative():
    """(a1,b1) o (a2,b2) = (a1 a2, a2 b1 + b2) composes two affine steps h -> a h + b; the
    decomposition above relies on it being associative (checked on random triples)."""
    rng = np.random.default_rng(8)
    op = lambda p, q: (p[0] * q[0], q[0] * p[1] + q[1])
    for _ in range(200):
        x, y, w = (tuple(rng.uniform(-2, 2, size=2)) for _ in range(3))
        l, r = op(op(x, y), w), op(x, op(y, w))
        assert np.allclose(l, r, rtol=1e-14, atol=1e-14)
        h = rng.standard_normal()
        assert np.isclose(l[0] * h + l[1], w[0] * (y[0] * (x[0] * h + x[1]) + y[1]) + w[1])


# ------------------------------------------------------------------------------------------
# P-h: decode steps reproduce prefill; a split prefill resumed from h_last equals the whole
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("bf16", [False, True])
def test_decode_steps_reproduce_prefill(bf16):
    rng = np.random.default_rng(9)
    c = rand_case(rng, batch=2, L=12, d_inner=3, N=4, bf16=bf16)
    kw = dict(D=c["D"], delta_bias=c["delta_bias"])
    out, h_last = oracle.scan_fwd(c["u"], c["delta"], c["A"], c["B"], c["C"], h0=c["h0"],
                                  z=c["z"], **kw)
    state = c["h0"].copy()
    for t in range(c["u"].shape[1]):
        o = oracle.state_update(state, c["u"][:, t], c["delta"][:, t], c["A"], c["B"][:, t],
                                c["C"][:, t], z=c["z"][:, t], **kw)
        np.testing.assert_allclose(o, out[:, t], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(state, h_last, rtol=1e-13, atol=1e-13)


def test_split_prefill_resumes_exactly():
    rng = np.random.default_rng(10)
    c = rand_case(rng, batch=2, L=40, d_inner=3, N=4)
    kw = dict(D=c["D"], z=c["z"], delta_bias=c["delta_bias"])
    whole, h_whole = oracle.scan_fwd(c["u"], c["delta"], c["A"], c["B"], c["C"], h0=c["h0"], **kw)
    for cut in (1, 17, 39):
        sl = lambda x, a, b: x[:, a:b]
        o1, h1 = oracle.scan_fwd(*(sl(c[k], 0, cut) for k in ("u", "delta")), c["A"],
                                 *(sl(c[k], 0, cut) for k in ("B", "C")), h0=c["h0"], D=c["D"],
                                 z=sl(c["z"], 0, cut), delta_bias=c["delta_bias"])
        o2, h2 = oracle.scan_fwd(*(sl(c[k], cut, 40) for k in ("u", "delta")), c["A"],
                                 *(sl(c[k], cut, 40) for k in ("B", "C")), h0=h1, D=c["D"],
                                 z=sl(c["z"], cut, 40), delta_bias=c["delta_bias"])
        np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), whole, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(h2, h_whole, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------------------------------
# P-i: linearity in (u, h0) for fixed dt (no gate) and causality
# ------------------------------------------------------------------------------------------
def test_linearity_and_causality():
    rng = np.random.default_rng(11)
    c = rand_case(rng, L=25)
    # inputs on a 1/64 grid so that the mixed input is exact in float32
    grid = lambda: (rng.integers(-512, 512, size=c["u"].shape) / 64.0).astype(np.float32)
    u1, u2 = grid(), grid()
    h01, h02 = rng.standard_normal(c["h0"].shape), rng.standard_normal(c["h0"].shape)
    al, be = 0.75, -1.25
    mix = (al * f64(u1) + be * f64(u2)).astype(np.float32)
    assert np.array_equal(f64(mix), al * f64(u1) + be * f64(u2))
    kw = dict(A=c["A"], B=c["B"], C=c["C"], D=c["D"], delta_bias=c["delta_bias"])
    o_mix, h_mix = oracle.scan_fwd(mix, c["delta"], h0=al * h01 + be * h02, **kw)
    o1, h1 = oracle.scan_fwd(u1, c["delta"], h0=h01, **kw)
    o2, h2 = oracle.scan_fwd(u2, c["delta"], h0=h02, **kw)
    np.testing.assert_allclose(o_mix, al * o1 + be * o2, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(h_mix, al * h1 + be * h2, rtol=1e-11, atol=1e-11)
    # causality: changing u at t0 leaves every earlier output bit-identical
    t0 = 13
    u_p = u1.copy()
    u_p[:, t0] += 3.0
    o_p, _ = oracle.scan_fwd(u_p, c["delta"], h0=h01, **kw)
    assert np.array_equal(o_p[:, :t0], o1[:, :t0])
    assert not np.allclose(o_p[:, t0], o1[:, t0])


# ------------------------------------------------------------------------------------------
# P-j: very large step with exact ZOH resets the state to its fixed point -B u / A
# ------------------------------------------------------------------------------------------
def test_large_step_resets_state_under_exact_zoh():
    rng = np.random.default_rng(12)
    c = rand_case(rng, L=6)
    A = -rng.uniform(1.0, 3.0, size=c["A"].shape).astype(np.float32)
    big = np.full_like(c["delta"], 60.0)
    _, h_last = oracle.scan_fwd(c["u"], big, A, c["B"], c["C"], delta_softplus=False,
                                h0=c["h0"], zoh_exact=True)
    want = -(c["B"][:, -1].astype(np.float64)[:, None, :] * c["u"][:, -1].astype(np.float64)[..., None]
             / A.astype(np.float64)[None])
    np.testing.assert_allclose(h_last, want, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------------------------------
# Marshalling: numpy twin agreement, row subsets, bf16 decode
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("zoh", [False, True])
@pytest.mark.parametrize("opts", ["all", "bare"])
def test_c_oracle_matches_numpy_twin(bf16, zoh, opts):
    rng = np.random.default_rng(13)
    c = rand_case(rng, batch=3, L=11, d_inner=5, N=6, bf16=bf16)
    kw = (dict(D=c["D"], z=c["z"], delta_bias=c["delta_bias"], h0=c["h0"]) if opts == "all"
          else dict(delta_softplus=False))
    if opts == "bare":
        c["delta"] = np.abs(widen(c["delta"])).astype(np.float32) if not bf16 else c["delta"] & 0x7FFF
    o_c, h_c = oracle.scan_fwd(c["u"], c["delta"], c["A"], c["B"], c["C"], zoh_exact=zoh, **kw)
    o_n, h_n = numpy_twin.scan_fwd(c["u"], c["delta"], c["A"], c["B"], c["C"], zoh_exact=zoh, **kw)
    np.testing.assert_allclose(o_c, o_n, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h_c, h_n, rtol=1e-12, atol=1e-12)


def test_row_subset_matches_full():
    rng = np.random.default_rng(14)
    c = rand_case(rng, batch=3, L=10, d_inner=7, N=4)
    kw = dict(D=c["D"], z=c["z"], delta_bias=c["delta_bias"], h0=c["h0"])
    full, h_full = oracle.scan_fwd(c["u"], c["delta"], c["A"], c["B"], c["C"], **kw)
    rows = np.array([20, 0, 8, 13, 7], dtype=np.int64)
    sub, h_sub = oracle.scan_fwd(c["u"], c["delta"], c["A"], c["B"], c["C"], rows=rows, **kw)
    for i, r in enumerate(rows):
        b, d = divmod(int(r), 7)
        assert np.array_equal(sub[i], full[b, :, d])
        assert np.array_equal(h_sub[i], h_full[b, d])
    state = c["h0"].copy()
    st_sub = c["h0"].copy()
    o_full = oracle.state_update(state, c["u"][:, 0], c["delta"][:, 0], c["A"], c["B"][:, 0],
                                 c["C"][:, 0], D=c["D"], z=c["z"][:, 0], delta_bias=c["delta_bias"])
    o_sub = oracle.state_update(st_sub, c["u"][:, 0], c["delta"][:, 0], c["A"], c["B"][:, 0],
                                c["C"][:, 0], D=c["D"], z=c["z"][:, 0], delta_bias=c["delta_bias"],
                                rows=rows)
    for i, r in enumerate(rows):
        b, d = divmod(int(r), 7)
        assert o_sub[i] == o_full[b, d]
        assert np.array_equal(st_sub[b, d], state[b, d])


def test_bf16_inputs_are_read_exactly():
    """The oracle's bf16 path must equal its fp32 path on the widened values (widened by torch's
    own bfloat16 conversion, a library routine independent of the oracle)."""
    rng = np.random.default_rng(15)
    c = rand_case(rng, batch=2, L=8, d_inner=3, N=4, bf16=True)
    kw = dict(D=c["D"], delta_bias=c["delta_bias"], h0=c["h0"])
    o_b, h_b = oracle.scan_fwd(c["u"], c["delta"], c["A"], c["B"], c["C"], z=c["z"], **kw)
    w = {k: widen(c[k]).astype(np.float32) for k in ("u", "delta", "B", "C", "z")}
    o_f, h_f = oracle.scan_fwd(w["u"], w["delta"], c["A"], w["B"], w["C"], z=w["z"], **kw)
    assert np.array_equal(o_b, o_f) and np.array_equal(h_b, h_f)


def test_bad_arguments_are_rejected():
    rng = np.random.default_rng(16)
    c = rand_case(rng)
    with pytest.raises(ValueError):
        oracle.scan_fwd(c["u"], c["delta"][:, :-1], c["A"], c["B"], c["C"])
    with pytest.raises(ValueError):
        oracle.scan_fwd(c["u"], c["delta"], c["A"], c["B"], c["C"], rows=np.array([10**6]))
