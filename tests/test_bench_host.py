"""Host logic of bench.py that runs without a GPU: the algorithmic byte and slot counts, the clock
settle rule, the traffic lookup's source check and the one-GPU guard."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from selective_state_space_36_amd import workloads as wl  # noqa: E402


def test_algorithmic_bytes_of_the_measured_layers():
    # 2.8B layer: u, delta, z, out at 2 B per element; B and C at 2 B per (b, t, n); A in
    # float32; D and the bias in float32
    w = wl.WORKLOADS[2]
    n = 4 * 4096 * 5120
    assert bench.prefill_bytes(w) == n * 8 + 2 * 4 * 4096 * 16 * 2 + 5120 * 16 * 4 + 2 * 5120 * 4
    assert bench.prefill_bytes(w) == 672_505_856
    # decode step: the float32 state read and written, u/delta/z/out, B/C, A, D, bias
    d = wl.WORKLOADS[4]
    assert bench.decode_bytes_per_step(d) == (8 * 128 * 5120 * 16 + 128 * 5120 * 8
                                              + 2 * 128 * 16 * 2 + 5120 * 16 * 4 + 2 * 5120 * 4)
    assert bench.decode_bytes_per_step(d) == 89_505_792
    # backward: 7 io tensors of the element count (u, delta, z, dout read; du, ddelta, dz
    # written), B/C read and dB/dC written, A and dA, D/bias and dD/dbias
    assert bench.backward_bytes(w) == (n * 7 * 2 + 4 * 4096 * 16 * (2 * 2 + 2 * 4)
                                       + 2 * 5120 * 16 * 4 + 4 * 5120 * 4)


def test_valu_slot_count():
    w = wl.WORKLOADS[2]
    assert bench.valu_slots(w) == w.elements * (16 * 6 + 19)
    assert bench.PEAK_VALU_SLOTS == pytest.approx(39.3216e12)


def test_exp_rate_is_per_second():
    w = wl.WORKLOADS[2]
    st = bench.exp_stats(w, 0.35)  # 350 us per call
    # 16 update exps + softplus + silu per element
    assert st["exp_per_element"] == 18
    assert st["exp_per_s"] == pytest.approx(w.elements * 18 / 350e-6, rel=1e-6)
    assert st["exp_frac"] == pytest.approx(w.elements * 18 / 350e-6 / (bench.PEAK_VALU_SLOTS / 2),
                                           abs=1e-4)
    assert 0.1 < st["exp_frac"] < 1.0


def test_backward_valu_slot_count():
    w = wl.WORKLOADS[2]
    given = bench.bwd_valu_slots(w, states_given=True)
    assert given == w.elements * (16 * 20 + 41)
    assert bench.bwd_valu_slots(w) == given + w.elements * (16 * 5 + 11)


def _fake_timer(monkeypatch, per_launch_ms):
    """bench.timed replaced by one that hands out the given per-launch times in order."""
    it = iter(per_launch_ms)
    calls = []

    def timed(torch, stream, fn, warmup, steps, per_launch=True):
        assert warmup == 0
        per = [next(it) for _ in range(steps)]
        calls.append(steps)
        return sum(per) / steps, per

    monkeypatch.setattr(bench, "timed", timed)
    return calls


def test_clock_settle_stops_once_the_launch_time_is_flat(monkeypatch):
    # falling by 5 % a block for 6 blocks, then flat
    times = []
    t = 0.50
    for _ in range(6):
        times += [t] * 10
        t *= 0.95
    times += [t] * 1000
    calls = _fake_timer(monkeypatch, times)
    means = bench.clock_settle(None, None, None)
    # block 7 is the first at the final time (still 5 % below block 6); the changes to blocks 8
    # and 9 are the first two under 1 %
    assert len(means) == 9 and sum(calls) == 90
    assert means[-1] == pytest.approx(t * 1e3)


def test_clock_settle_runs_at_least_the_minimum(monkeypatch):
    calls = _fake_timer(monkeypatch, [0.4] * 1000)
    means = bench.clock_settle(None, None, None)
    assert sum(calls) == 60 and len(means) == 6


def test_clock_settle_is_capped(monkeypatch):
    # never flat: alternating 0.40 / 0.42 ms blocks
    times = []
    for i in range(100):
        times += [0.40 if i % 2 == 0 else 0.42] * 10
    calls = _fake_timer(monkeypatch, times)
    means = bench.clock_settle(None, None, None)
    assert sum(calls) == 400 and len(means) == 40


def test_traffic_is_reported_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    name = "mamba2.8b-prefill"
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # a copy of the kernel sources under the patched root, which the hash is taken over
    csrc = tmp_path / "selective_state_space_36_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.KERNEL_SOURCES[name]:
        src = os.path.join(ROOT, "selective_state_space_36_amd", "csrc", f)
        (csrc / f).write_bytes(open(src, "rb").read())
    good = bench.kernel_source_hash(name)
    body = "source_hash: {}\nhbm_bytes_per_launch: 675619628\n"
    (prof / f"traffic_{name}.txt").write_text(body.format(good))
    assert bench.measured_traffic(name) == 675619628
    (prof / f"traffic_{name}.txt").write_text(body.format("0" * 16))
    assert bench.measured_traffic(name) is None
    # a changed source invalidates the stored figure
    (prof / f"traffic_{name}.txt").write_text(body.format(good))
    first = bench.KERNEL_SOURCES[name][0]
    (csrc / first).write_bytes((csrc / first).read_bytes() + b"\n// changed\n")
    assert bench.measured_traffic(name) is None
    # no summary at all
    (prof / f"traffic_{name}.txt").unlink()
    assert bench.measured_traffic(name) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
