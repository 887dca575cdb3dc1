"""The pins must bite: plant plausible mistakes in a copy of the oracle's C source (on the CPU),
build each copy, and check that at least one pin fails for every one of them."""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_bwd as bwd_pins
from tests import test_oracle_conv as conv_pins
from tests import test_oracle_pins as pins
from tests import test_oracle_scan2 as scan2_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ss_oracle.c")

# (name, original text, planted mistake)
MUTATIONS = [
    ("y from h before the update",
     "        h[n] = abar * h[n] + bbar * x;\n        y += rd(C, bc + n, io_dtype) * h[n];",
     "        y += rd(C, bc + n, io_dtype) * h[n];\n        h[n] = abar * h[n] + bbar * x;"),
    ("bias after softplus",
     "  double s = raw + (delta_bias ? (double)delta_bias[d] : 0.0);\n  return delta_softplus ? softplus(s) : s;",
     "  double s = raw;\n  return (delta_softplus ? softplus(s) : s) + (delta_bias ? (double)delta_bias[d] : 0.0);"),
    ("D outside the gate",
     "      if (D) y += (double)D[d] * x;\n      if (z) y *= silu(rd(z, e, io_dtype));",
     "      if (z) y *= silu(rd(z, e, io_dtype));\n      if (D) y += (double)D[d] * x;"),
    ("decay sign flipped", "double abar = exp(dt * a);\n        double bbar",
     "double abar = exp(-dt * a);\n        double bbar"),
    ("skip term dropped", "      if (D) y += (double)D[d] * x;\n      if (z) y *= silu(rd(z, e, io_dtype));\n      out[i",
     "      if (z) y *= silu(rd(z, e, io_dtype));\n      out[i"),
    ("input not scaled by dt", "  if (!zoh_exact) return dt;", "  if (!zoh_exact) return 1.0;"),
    ("B and C swapped", "        y += rd(C, bc + n, io_dtype) * h[n];", "        y += rd(B, bc + n, io_dtype) * h[n];"),
    ("A transposed", "        double a = (double)A[d * d_state + n];\n        double abar",
     "        double a = (double)A[(n * d_inner + d) % (d_inner * d_state)];\n        double abar"),
    ("exact ZOH without expm1", "  return expm1(dt * a) / a;", "  return exp(dt * a) / a;"),
    ("initial state ignored", "    for (int64_t n = 0; n < d_state; ++n) h[n] = h0 ? h0[r * d_state + n] : 0.0;",
     "    for (int64_t n = 0; n < d_state; ++n) h[n] = 0.0;"),
    ("gate is sigmoid not silu", "static double silu(double z) { return z / (1.0 + exp(-z)); }",
     "static double silu(double z) { return 1.0 / (1.0 + exp(-z)); }"),
    ("softplus without the max", "return (s > 0.0 ? s : 0.0) + log1p(exp(-fabs(s)));",
     "return log1p(exp(-fabs(s)));"),
    ("B indexed by channel", "double bbar = bbar_factor(dt, a, zoh_exact) * rd(B, bc + n, io_dtype);",
     "double bbar = bbar_factor(dt, a, zoh_exact) * rd(B, (b * seqlen + t) * d_state + (n + d) % d_state, io_dtype);"),
    ("decode state not written back", "      *h = exp(dt * a) * (*h) + bbar_factor",
     "      double hn = exp(dt * a) * (*h) + bbar_factor"),
    ("chunk carry dropped", "          y += rd(C, bc + n, io_dtype) * (hloc[n] + prod[n] * h_in[n]);",
     "          y += rd(C, bc + n, io_dtype) * hloc[n];"),
    ("conv taps reversed", "          int64_t ts = t - (k - 1) + j;", "          int64_t ts = t - j;"),
    ("conv bias dropped", "        double acc = conv_b ? (double)conv_b[d] : 0.0;",
     "        double acc = 0.0;"),
    ("conv history ignored",
     "            xv = x_prev ? rd(x_prev, (b * (k - 1) + (k - 1) + ts) * d_inner + d, io_dtype) : 0.0;",
     "            xv = 0.0;"),
    ("conv without silu", "        u[(b * seqlen + t) * d_inner + d] = silu(acc);",
     "        u[(b * seqlen + t) * d_inner + d] = acc;"),
    ("adjoint without decay",
     "      lam[n] = gy * cn + (t == seqlen - 1 ? lam[n] : e_next[n] * lam[n]);",
     "      lam[n] = gy * cn + lam[n];"),
    ("softplus derivative dropped", "    double dd = delta_softplus ? ddt / (1.0 + exp(-s)) : ddt;",
     "    double dd = ddt;"),
    ("dC from the previous state", "      dC[bc + n] += gy * h[n];", "      dC[bc + n] += gy * hp[n];"),
    ("dA without the decay factor", "      dA[d * d_state + n] += lam[n] * dt * et * hp[n];",
     "      dA[d * d_state + n] += lam[n] * dt * hp[n];"),
    ("gate derivative without the z term",
     "      if (dz) dz[e] = dout[e] * y * sg * (1.0 + zv * (1.0 - sg));",
     "      if (dz) dz[e] = dout[e] * y * sg;"),
    ("head reads the wrong group", "    int64_t b = r / nheads, h = r % nheads, g = h / hpg;",
     "    int64_t b = r / nheads, h = r % nheads, g = h % ngroups;"),
    ("multi-head decay after the input",
     "          hs[n * headdim + p] = decay * hs[n * headdim + p] + bn * rd(x, xo + p, io_dtype);",
     "          hs[n * headdim + p] = decay * (hs[n * headdim + p] + bn * rd(x, xo + p, io_dtype));"),
    ("multi-head y before the update",
     "        for (int64_t n = 0; n < d_state; ++n) y += rd(C, bc + n, io_dtype) * hs[n * headdim + p];",
     "        for (int64_t n = 0; n < d_state; ++n) y += rd(C, bc + n, io_dtype) * hs[n * headdim + p] / decay;"),
    ("conv looks ahead", "          if (ts >= 0)\n            xv = rd(x, (b * seqlen + ts) * d_inner + d, io_dtype);",
     "          if (ts >= 0)\n            xv = rd(x, (b * seqlen + (ts + 1 < seqlen ? ts + 1 : ts)) * d_inner + d, io_dtype);"),
    ("exact-ZOH gradient ignores the gain", "      double g = bbar_factor(dt, a, zoh_exact);",
     "      double g = dt;"),
    ("exact-ZOH gain's dt derivative dropped", "      double g_dt = zoh_exact ? et : 1.0;",
     "      double g_dt = 1.0;"),
    ("exact-ZOH input term of dA dropped",
     "      if (zoh_exact) dA[d * d_state + n] += lam[n] * zoh_gain_da(dt, a, et) * bn * x;\n", ""),
    ("exact-ZOH dA limit at a = 0", "  if (a == 0.0) return 0.5 * dt * dt;", "  if (a == 0.0) return dt * dt;"),
    ("summed gradient partial of one thread dropped",
     "      for (int th = 0; th < nthreads; ++th) acc += part",
     "      for (int th = 1; th < nthreads; ++th) acc += part"),
]

PIN_CALLS = [
    lambda: scan2_pins.test_equals_mamba1_with_constant_A_rows(False),
    scan2_pins.test_quadratic_dual_form,
    scan2_pins.test_group_sharing,
    lambda: bwd_pins.test_gradients_match_finite_differences(True),
    lambda: bwd_pins.test_gradients_match_finite_differences(False),
    lambda: bwd_pins.test_exact_zoh_gradients_match_finite_differences(True),
    bwd_pins.test_exact_zoh_gradient_at_zero_decay,
    bwd_pins.test_summed_gradients_do_not_depend_on_thread_count,
    bwd_pins.test_decay_free_linear_closed_form,
    lambda: conv_pins.test_matches_numpy_convolution(4, False, True),
    lambda: conv_pins.test_matches_numpy_convolution(2, True, False),
    conv_pins.test_last_tap_only_is_pointwise_silu,
    conv_pins.test_first_tap_only_is_a_delay,
    conv_pins.test_causal,
    lambda: pins.test_golden_worked_examples("gated_rnn", False),
    lambda: pins.test_golden_worked_examples("gated_rnn", True),
    lambda: pins.test_golden_worked_examples("sum_and_reset", False),
    lambda: pins.test_golden_worked_examples("sum_and_reset", True),
    pins.test_zero_step_gives_skip_only_exactly,
    lambda: pins.test_time_invariant_equals_convolution(True),
    pins.test_no_decay_is_prefix_sum,
    pins.test_pure_decay_of_initial_state,
    pins.test_gated_rnn_special_case,
    lambda: pins.test_unrolled_brute_force(False),
    lambda: pins.test_unrolled_brute_force(True),
    lambda: pins.test_chunked_equals_sequential(16),
    lambda: pins.test_decode_steps_reproduce_prefill(False),
    pins.test_split_prefill_resumes_exactly,
    pins.test_large_step_resets_state_under_exact_zoh,
]


@pytest.mark.parametrize("name,orig,bad", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, orig, bad, tmp_path):
    src = open(SRC).read()
    # a mutation may legitimately apply to the decode/chunked copy only; require one hit
    assert src.count(orig) >= 1, f"mutation anchor not found: {name}"
    mutated = src.replace(orig, bad, 1)
    if name == "decode state not written back":
        mutated = mutated.replace(
            "      y += rd(C, b * d_state + n, io_dtype) * (*h);",
            "      y += rd(C, b * d_state + n, io_dtype) * hn;", 1)
    c_path = tmp_path / "m.c"
    so_path = tmp_path / "libm.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-o", str(so_path),
                    str(c_path), "-lm"], check=True, capture_output=True)
    prev = oracle.use_library(str(so_path))
    try:
        caught = []
        for call in PIN_CALLS:
            try:
                call()
            except (AssertionError, ValueError):
                caught.append(call)
        assert caught, f"no pin caught the planted mistake: {name}"
    finally:
        oracle.restore_library(prev)


def test_unmutated_source_passes_every_pin():
    for call in PIN_CALLS:
        call()
