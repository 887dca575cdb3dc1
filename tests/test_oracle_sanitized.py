"""The oracle's C source under AddressSanitizer and UndefinedBehaviorSanitizer (host code only).

ss_oracle.c is built with gcc -fsanitize=address,undefined (every undefined-behaviour check
fatal), loaded into a child Python process with the ASan runtime preloaded, and every pin of the
oracle runs against that build, plus calls on row subsets, empty sizes and wide states.  Any
out-of-bounds access, use after free, signed overflow or misaligned load aborts the child and
fails the test."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(os.path.dirname(oracle.__file__), "ss_oracle.c")

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import numpy as np
import oracle
oracle.use_library({lib!r})
from tests import test_oracle_mutations as m
for call in m.PIN_CALLS:
    call()
from tests import test_oracle_pins as pins
from tests import test_oracle_bwd as bwd
from tests import test_oracle_conv as conv
bwd.test_without_gate_skip_bias_or_h0()
bwd.test_empty_sequence_passes_dh_last_to_dh0()
bwd.test_exact_zoh_gradients_match_finite_differences(False)
from selective_state_space_36_amd import workloads as wl
w = wl.WORKLOADS[1]
p = wl.make_prefill(w, batch=2, seqlen=70, d_inner=40, seed=3)
rows = np.array([0, 39, 40, 79], dtype=np.int64)
full, fh = oracle.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["D"], z=p["z"],
                           delta_bias=p["delta_bias"])
sub, sh = oracle.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["D"], z=p["z"],
                          delta_bias=p["delta_bias"], rows=rows)
assert np.array_equal(sub, full.transpose(0, 2, 1).reshape(-1, 70)[rows])
# wide state (64) and a one-state case through every entry point
for N in (1, 64):
    rng = np.random.default_rng(N)
    u = rng.standard_normal((1, 9, 3)).astype(np.float32)
    dl = (0.3 * rng.standard_normal((1, 9, 3))).astype(np.float32)
    A = -rng.uniform(0.5, 2, (3, N)).astype(np.float32)
    B = rng.standard_normal((1, 9, N)).astype(np.float32)
    C = rng.standard_normal((1, 9, N)).astype(np.float32)
    oracle.scan_fwd(u, dl, A, B, C, zoh_exact=True)
    oracle.scan_fwd_chunked(u, dl, A, B, C, 4)
    oracle.scan_bwd(u, dl, A, B, C, np.ones((1, 9, 3)), zoh_exact=True)
    st = rng.standard_normal((1, 3, N))
    oracle.state_update(st, u[:, 0], dl[:, 0], A, B[:, 0], C[:, 0])
# empty sizes
e = np.zeros((0, 5, 3), np.float32)
oracle.scan_fwd(e, e, np.zeros((3, 4), np.float32), np.zeros((0, 5, 4), np.float32),
                np.zeros((0, 5, 4), np.float32))
print("sanitized pins ok")
"""


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not asan or not os.path.exists(asan):
        pytest.skip("gcc has no ASan runtime here")
    lib = tmp_path / "libss_oracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-shared", "-fPIC",
                    "-std=c99", "-Wall", "-Werror", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-o", str(lib), SRC, "-lm"],
                   check=True, capture_output=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    # Python's own allocations are not this test's business; aborting on the first report is
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, lib=str(lib))], env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "sanitized pins ok" in r.stdout, (
        f"sanitized oracle run failed (rc {r.returncode}):\n{r.stdout[-3000:]}\n"
        f"{r.stderr[-6000:]}")
