"""Benchmark of the selective scan (S6) on one MI355X.

Prints ONE JSON line.  A step is one prefill call (ss_scan_fwd) on the Mamba-2.8B-shaped layer
(batch 4, L 4096, d_inner 5120, d_state 16, bf16 io, silu gate, fp32 state) with inputs resident
in HBM; `value` is B*L*D elements per second over K timed steps.  The same line carries:
  * roofline: the prefill kernel against the VALU issue rate (on gfx950 its 115 VALU slots per
    element take longer than its 8 bytes of HBM traffic), with the HBM view alongside;
  * decode: the batch-128 single-token step (ss_state_update) run 1000 times back to back over
    pre-generated inputs: end-to-end us/step, kernel-only us/step and state GB/s;
  * cpu_baseline: the fp64 C oracle timed on this host's cores on a bounded sample of rows.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--decode-steps 1000]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0     # dense bf16 MFMA, MI355X
# VALU issue slots per second: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (one 64-lane wave op
# every 4 cycles per SIMD).  Non-packed fp32 ops take one slot; v_exp_f32 takes two on gfx950.
PEAK_VALU_SLOTS = 256 * 4 * 16 * 2.4e9
SLOTS_PER_UPDATE = 6          # 1 exp (2 slots) + dt*A, (dt*u)*B, state FMA, C.h FMA
SLOTS_PER_ELEMENT_GATED = 19  # bias add, softplus (exp 2 + log 4 + add), dt*u, skip FMA,
                              # silu (exp 2 + add + rcp 4 + mul), gate mul
SLOTS_PER_ELEMENT_PLAIN = 10


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # ~40 ms of warm-up by default: under sustained load of this kernel the clock dips over the
    # first ~20 launches and settles after ~40 (measured per launch: ~400 us, then 450-510 us,
    # then 355-375 us), and the timed steps are meant to see the steady state.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3])
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-multihead", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    return ap.parse_args()


def calibrate_copy(torch):
    """A plain copy of known size: reads and writes exactly 1 GiB.  Its FETCH_SIZE/WRITE_SIZE
    under rocprofv3 --pmc give the factor that converts those counters into HBM bytes."""
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n, "launches": 3}))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# Sources each measured kernel is built from: a counter summary under profiles/ stays valid only
# while these files are unchanged.
# untimed calls before each section after the main one: switching to another kernel moves the
# clock again for a few launches
SECTION_WARMUP = 20

KERNEL_SOURCES = {
    "mamba2.8b-prefill": ["ss_device.h", "ss_launch.h", "ss_scan_kernel.h", "ss_scan_fwd.hip"],
    "decode-b128": ["ss_device.h", "ss_launch.h", "ss_state_update.hip"],
    "mamba2-80h-prefill": ["ss_device.h", "ss_scan2.h", "ss_scan2_mfma.hip"],
}


def kernel_source_hash(name: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_36_amd", "csrc")
    for fname in sorted(KERNEL_SOURCES[name]):
        with open(os.path.join(csrc, fname), "rb") as f:
            h.update(fname.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(name: str):
    """HBM bytes per launch of the named kernel/workload from the committed rocprofv3 counter
    summary profiles/traffic_<name>.txt, if it was taken on the current kernel sources;
    otherwise None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            key, sep, val = line.partition(":")
            if sep:
                vals[key.strip()] = val.strip()
    if vals.get("source_hash") != kernel_source_hash(name):
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def prefill_bytes(w) -> int:
    s = 2 if w.io_dtype == "bf16" else 4
    per_elem = (4 if w.gate else 3) * s          # u, delta, (z), out
    return (w.elements * per_elem + 2 * w.batch * w.seqlen * w.d_state * s
            + w.d_inner * w.d_state * 4 + 2 * w.d_inner * 4)


def decode_bytes_per_step(w) -> int:
    s = 2
    return (8 * w.batch * w.d_inner * w.d_state + w.batch * w.d_inner * 4 * s
            + 2 * w.batch * w.d_state * s + w.d_inner * w.d_state * 4 + 2 * w.d_inner * 4)


def dev(x, torch, np):
    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def bench_prefill(args, torch, np, ops, wl):
    w = wl.WORKLOADS[args.workload]
    log(f"generating {w.name} inputs")
    p = wl.make_prefill(w)
    u, dl, A, B, C = (dev(p[k], torch, np) for k in ("u", "delta", "A", "B", "C"))
    D, z, db = dev(p["D"], torch, np), dev(p["z"], torch, np), dev(p["delta_bias"], torch, np)
    out = torch.empty_like(u)
    nbytes = ops.workspace_bytes(w.batch, w.seqlen, w.d_inner, w.d_state, u.dtype)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        ops.scan_fwd(u, dl, A, B, C, D=D, z=z, delta_bias=db, out=out, workspace=ws,
                     stream=stream)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # per-launch events over the timed region give the kernel's average duration
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_all0, t_all1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record(stream)
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    t_all1.record(stream)
    torch.cuda.synchronize()
    ms_total = t_all0.elapsed_time(t_all1)
    per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    ms_step = ms_total / args.steps
    ms_kernel = sum(per) / len(per)
    log(f"prefill {ms_step * 1e3:.1f} us/step (kernel avg {ms_kernel * 1e3:.1f} us, "
        f"min {per[0] * 1e3:.1f})")

    # the same layer with the exact zero-order-hold input term (SS_FLAG_ZOH_EXACT)
    zoh_out = torch.empty_like(u)
    zsteps = max(3, args.steps // 4)
    for _ in range(SECTION_WARMUP):
        ops.scan_fwd(u, dl, A, B, C, D=D, z=z, delta_bias=db, out=zoh_out, workspace=ws,
                     zoh_exact=True, stream=stream)
    torch.cuda.synchronize()
    zs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(zsteps)]
    for a_, b_ in zs:
        a_.record(stream)
        ops.scan_fwd(u, dl, A, B, C, D=D, z=z, delta_bias=db, out=zoh_out, workspace=ws,
                     zoh_exact=True, stream=stream)
        b_.record(stream)
    torch.cuda.synchronize()
    ms_zoh = sum(a_.elapsed_time(b_) for a_, b_ in zs) / zsteps
    log(f"prefill exact-hold kernel avg {ms_zoh * 1e3:.1f} us")

    # the same layer with the block's front end fused in (ss_scan_fwd_conv): the benchmark's u
    # plays x, and u = silu(causal depthwise conv of width 4 + bias) is formed in the kernel
    g = torch.Generator(device="cuda").manual_seed(77)
    cw = 0.5 * torch.randn((w.d_inner, 4), device="cuda", generator=g)
    cbias = 0.2 * torch.randn((w.d_inner,), device="cuda", generator=g)
    conv_out = torch.empty_like(u)
    for _ in range(SECTION_WARMUP):
        ops.scan_fwd_conv(u, cw, cbias, dl, A, B, C, D=D, z=z, delta_bias=db, out=conv_out,
                          workspace=ws, stream=stream)
    torch.cuda.synchronize()
    cs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(zsteps)]
    for a_, b_ in cs:
        a_.record(stream)
        ops.scan_fwd_conv(u, cw, cbias, dl, A, B, C, D=D, z=z, delta_bias=db, out=conv_out,
                          workspace=ws, stream=stream)
        b_.record(stream)
    torch.cuda.synchronize()
    ms_conv = sum(a_.elapsed_time(b_) for a_, b_ in cs) / zsteps
    log(f"prefill with fused conv front end kernel avg {ms_conv * 1e3:.1f} us")

    # the backward (ss_scan_bwd) of the same layer for a random upstream gradient
    dout = torch.randn(u.shape, device="cuda", generator=g).to(u.dtype)
    nbw = int(ops.lib().ss_scan_bwd_workspace_bytes(w.batch, w.seqlen, w.d_inner, w.d_state,
                                                     ops.SS_BF16 if w.io_dtype == "bf16"
                                                     else ops.SS_F32))
    ws_b = torch.empty(max(nbw, 1), dtype=torch.uint8, device="cuda")
    for _ in range(SECTION_WARMUP // 4):
        ops.scan_bwd(u, dl, A, B, C, dout, D=D, z=z, delta_bias=db, workspace=ws_b,
                     stream=stream)
    torch.cuda.synchronize()
    bsteps = max(2, args.steps // 10)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(bsteps):
        ops.scan_bwd(u, dl, A, B, C, dout, D=D, z=z, delta_bias=db, workspace=ws_b,
                     stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_bwd = e0.elapsed_time(e1) / bsteps
    log(f"backward {ms_bwd * 1e3:.1f} us per call")
    del ws_b
    # the training path: the forward saving its chunk-end states (ss_scan_fwd_states), then the
    # backward taking them (SS_FLAG_STATES_GIVEN) instead of rerunning the forward
    st_buf = torch.empty((w.batch, (w.seqlen + 15) // 16, w.d_inner, w.d_state),
                         dtype=torch.float32, device="cuda")
    st_out = torch.empty_like(u)
    fwd_s = lambda: ops.scan_fwd_states(u, dl, A, B, C, D=D, z=z, delta_bias=db, out=st_out,
                                        states=st_buf, workspace=ws, stream=stream)
    bwd_s = lambda: ops.scan_bwd(u, dl, A, B, C, dout, D=D, z=z, delta_bias=db, states=st_buf,
                                 stream=stream)
    for _ in range(SECTION_WARMUP // 4):
        fwd_s()
        bwd_s()
    torch.cuda.synchronize()
    times = {}
    for name, fn in (("fwd", fwd_s), ("bwd", bwd_s)):
        e0.record(stream)
        for _ in range(bsteps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times[name] = e0.elapsed_time(e1) / bsteps
    train = dict(ms_fwd_states=times["fwd"], ms_bwd_states=times["bwd"])
    log(f"forward saving states {times['fwd'] * 1e3:.1f} us, backward given them "
        f"{times['bwd'] * 1e3:.1f} us")
    del st_buf, st_out

    # spot parity check of the benchmarked output on a few rows
    import oracle
    rows = np.array([0, 1, w.d_inner - 1, (w.batch - 1) * w.d_inner + w.d_inner // 2],
                    dtype=np.int64)
    g = out.float()[torch.from_numpy(rows // w.d_inner).cuda(), :,
                    torch.from_numpy(rows % w.d_inner).cuda()].cpu().numpy().astype(np.float64)
    r, _ = oracle.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["D"], z=p["z"],
                           delta_bias=p["delta_bias"], rows=rows)
    err = np.abs(g - r)
    ok = bool(np.all(err <= 2e-2 + 2e-2 * np.abs(r)))
    gz = zoh_out.float()[torch.from_numpy(rows // w.d_inner).cuda(), :,
                         torch.from_numpy(rows % w.d_inner).cuda()].cpu().numpy().astype(np.float64)
    rz, _ = oracle.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["D"], z=p["z"],
                            delta_bias=p["delta_bias"], rows=rows, zoh_exact=True)
    errz = np.abs(gz - rz)
    ok = ok and bool(np.all(errz <= 2e-2 + 2e-2 * np.abs(rz)))
    # fused front end: oracle conv_silu on the sampled rows' channels, then the scan
    sel_b, sel_d = rows // w.d_inner, rows % w.d_inner
    cw_h, cb_h = cw.cpu().numpy(), cbias.cpu().numpy()
    gc = conv_out.float()[torch.from_numpy(sel_b).cuda(), :,
                          torch.from_numpy(sel_d).cuda()].cpu().numpy().astype(np.float64)
    errc = 0.0
    for i, (bi, di) in enumerate(zip(sel_b, sel_d)):
        one = lambda k: np.ascontiguousarray(p[k][bi:bi + 1, :, di:di + 1])
        uc = oracle.conv_silu(one("u"), cw_h[di:di + 1], cb_h[di:di + 1])
        rc, _ = oracle.scan_fwd(uc, one("delta"), p["A"][di:di + 1],
                                np.ascontiguousarray(p["B"][bi:bi + 1]),
                                np.ascontiguousarray(p["C"][bi:bi + 1]), D=p["D"][di:di + 1],
                                z=one("z"), delta_bias=p["delta_bias"][di:di + 1])
        e = np.abs(gc[i] - rc[0, :, 0])
        ok = ok and bool(np.all(e <= 2e-2 + 2e-2 * np.abs(rc[0, :, 0])))
        errc = max(errc, float(e.max()))
    return (w, p, ms_step, ms_kernel, ms_zoh, ms_conv, ms_bwd, train, ok,
            float(max(err.max(), errz.max(), errc)))


def bench_decode(args, torch, np, ops, wl):
    w = wl.WORKLOADS[4]
    steps = args.decode_steps
    log(f"generating {steps} decode steps")
    d = wl.make_decode(w, steps=steps)
    st = dev(d["state"], torch, np)
    u, dl, z, B, C = (dev(d[k], torch, np) for k in ("u", "delta", "z", "B", "C"))
    A, D, db = dev(d["A"], torch, np), dev(d["D"], torch, np), dev(d["delta_bias"], torch, np)
    out = torch.empty((steps, w.batch, w.d_inner), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def one(s):
        ops.state_update(st, u[s], dl[s], A, B[s], C[s], D=D, z=z[s], delta_bias=db, out=out[s],
                         stream=stream)

    for s in range(min(20, steps)):
        one(s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(steps):
        one(s)
    e1.record(stream)
    torch.cuda.synchronize()
    us_e2e = e0.elapsed_time(e1) * 1e3 / steps
    # kernel-only: events around each launch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for s in range(steps):
        ev[s][0].record(stream)
        one(s)
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    us_kernel = sum(per) / len(per)
    log(f"decode {us_e2e:.2f} us/step end-to-end, kernel {us_kernel:.2f} us (median "
        f"{per[len(per) // 2]:.2f})")

    # the same launches captured once into a HIP graph and replayed (launch gaps shrink)
    gsteps = min(steps, 200)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        for s in range(gsteps):  # warm the capture stream once outside the graph
            ops.state_update(st, u[s], dl[s], A, B[s], C[s], D=D, z=z[s], delta_bias=db,
                             out=out[s], stream=cap)
        cap.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            for s in range(gsteps):
                ops.state_update(st, u[s], dl[s], A, B[s], C[s], D=D, z=z[s], delta_bias=db,
                                 out=out[s], stream=cap)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // gsteps)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us_graph = e0.elapsed_time(e1) * 1e3 / (reps * gsteps)
    del graph

    # cold: 8 state buffers used in turn (8 x 41.9 MB > the 256 MB Infinity Cache), as 8 layers
    # of a model would, so every step streams its state from HBM
    nbuf = 8
    states = [st.clone() for _ in range(nbuf)]

    def one_cold(s):
        ops.state_update(states[s % nbuf], u[s], dl[s], A, B[s], C[s], D=D, z=z[s],
                         delta_bias=db, out=out[s], stream=stream)

    for s in range(min(2 * nbuf, steps)):
        one_cold(s)
    torch.cuda.synchronize()
    e0.record(stream)
    for s in range(steps):
        one_cold(s)
    e1.record(stream)
    torch.cuda.synchronize()
    us_cold = e0.elapsed_time(e1) * 1e3 / steps
    del states

    # inputs reused: the same step's u, delta, z, B, C every time (cache- and TLB-resident),
    # which isolates the state stream from the cost of touching fresh input pages each step
    for s in range(20):
        one(0)
    torch.cuda.synchronize()
    e0.record(stream)
    for s in range(steps):
        one(0)
    e1.record(stream)
    torch.cuda.synchronize()
    us_hot = e0.elapsed_time(e1) * 1e3 / steps
    log(f"decode graph {us_graph:.2f} us/step, cold (8 rotating states) {us_cold:.2f} us/step, "
        f"inputs reused {us_hot:.2f} us/step")

    # the step with the width-4 front end fused in (ss_state_update_conv): u is formed from
    # the block's x (u[s] here) and a (batch, 3, d_inner) window updated in place
    k = 4
    rng = np.random.default_rng(44)
    cw = torch.from_numpy((0.5 * rng.standard_normal((w.d_inner, k))).astype(np.float32)).cuda()
    cb = torch.from_numpy((0.2 * rng.standard_normal(w.d_inner)).astype(np.float32)).cuda()
    cs = torch.zeros((w.batch, k - 1, w.d_inner), dtype=torch.bfloat16, device="cuda")

    def one_conv(s):
        ops.state_update_conv(st, cs, u[s], cw, cb, dl[s], A, B[s], C[s], D=D, z=z[s],
                              delta_bias=db, out=out[s], stream=stream)

    for s in range(min(20, steps)):
        one_conv(s)
    torch.cuda.synchronize()
    e0.record(stream)
    for s in range(steps):
        one_conv(s)
    e1.record(stream)
    torch.cuda.synchronize()
    us_conv = e0.elapsed_time(e1) * 1e3 / steps
    log(f"decode with fused front end {us_conv:.2f} us/step")
    nb = decode_bytes_per_step(w)
    return dict(
        workload=w.name, batch=w.batch, d_inner=w.d_inner, d_state=w.d_state, steps=steps,
        us_per_step_end_to_end=round(us_e2e, 3), us_per_step_kernel=round(us_kernel, 3),
        us_per_step_kernel_median=round(per[len(per) // 2], 3),
        state_GBps=round(8 * w.batch * w.d_inner * w.d_state / (us_e2e * 1e-6) / 1e9, 1),
        # roofline over the back-to-back timed region (events around all steps): events
        # around each launch add about 2 us of their own, so us_per_step_kernel reads high
        roofline=dict(bound="hbm", achieved=round(nb / (us_e2e * 1e-6) / 1e9, 1),
                      peak=PEAK_HBM_GBPS, unit="GB/s",
                      frac=round(nb / (us_e2e * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                      traffic=measured_traffic(w.name), kernel_us=round(us_e2e, 3)),
        us_per_step_graph=round(us_graph, 3),
        inputs_reused=dict(us_per_step_end_to_end=round(us_hot, 3),
                           state_GBps=round(8 * w.batch * w.d_inner * w.d_state / (us_hot * 1e-6)
                                            / 1e9, 1)),
        cold=dict(us_per_step_end_to_end=round(us_cold, 3), state_buffers=nbuf,
                  achieved_GBps=round(nb / (us_cold * 1e-6) / 1e9, 1),
                  frac=round(nb / (us_cold * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)),
        conv_front_end=dict(us_per_step_end_to_end=round(us_conv, 3), conv_k=k,
                            note="ss_state_update_conv: width-4 causal conv + SiLU on x and the "
                                 "in-place window shift fused into the step"),
        note="warm: one state (41.9 MB) resident across steps, which fits the 256 MB Infinity "
             "Cache; cold: 8 states used in turn")


def bench_multihead(args, torch, np, ops, wl):
    """The multi-head scalar-transition scan (ss_scan2_fwd) on the Mamba-2-shaped layer: bf16
    with headdim 64 and d_state 128 runs the chunked dual form on the matrix cores.  Its floor is
    HBM (the algorithmic bytes at 8 TB/s); the MFMA work is reported alongside."""
    w = wl.MULTIHEAD
    log(f"generating {w.name} inputs")
    p = wl.make_multihead(w)
    x, dt, z, B, C = (dev(p[k], torch, np) for k in ("x", "dt", "z", "B", "C"))
    A, D, db = (dev(p[k], torch, np) for k in ("A", "D", "dt_bias"))
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    run = lambda: ops.scan2_fwd(x, dt, A, B, C, D=D, z=z, dt_bias=db, out=out, stream=stream)
    for _ in range(SECTION_WARMUP):
        run()
    torch.cuda.synchronize()
    steps = max(3, args.steps // 4)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a_, b_ in ev:
        a_.record(stream)
        run()
        b_.record(stream)
    torch.cuda.synchronize()
    ms = sum(a_.elapsed_time(b_) for a_, b_ in ev) / steps
    log(f"multi-head scan {ms * 1e3:.1f} us per call")
    # spot parity on two heads against the oracle
    import oracle
    heads = np.array([0, w.nheads - 1])
    sub = lambda a: np.ascontiguousarray(a[:, :, heads])
    ro, _ = oracle.scan2_fwd(sub(p["x"]), sub(p["dt"]), p["A"][heads], p["B"], p["C"],
                             D=p["D"][heads], z=sub(p["z"]), dt_bias=p["dt_bias"][heads])
    go = out[:, :, torch.from_numpy(heads).cuda()].float().cpu().numpy().astype(np.float64)
    err = np.abs(go - ro)
    ok = bool(np.all(err <= 2e-2 + 2e-2 * np.abs(ro)))
    N, P, Q = w.d_state, w.headdim, 64
    nbytes = 3 * w.elements * 2 + w.batch * w.seqlen * w.nheads * 2 \
        + 2 * w.batch * w.seqlen * w.ngroups * N * 2 + 3 * w.nheads * 4
    # dense products of the chunked form per (batch, head, 64-step chunk): the 10 causal 16x16
    # tiles of C B^T (K = N) and of M X (K = 16 per tile pair), the state update B^T (w o X) and
    # C S_in; "executed" counts the second (low-part) product of each split fp32 operand
    chunks = w.batch * w.nheads * ((w.seqlen + Q - 1) // Q)
    cb, mx = 10 * 16 * 16 * N * 2, 10 * 16 * 16 * 16 * 2 * P // 16
    st, yo = 2 * N * Q * P, 2 * Q * N * P
    flops = chunks * (cb + mx + st + yo)
    mx_exec = 192 * 16 * P * 2  # M X runs in 32-wide K blocks: 32 + 32 + 64 + 64 per t-tile
    flops_exec = chunks * (cb + 2 * mx_exec + 2 * st + 2 * yo)
    sec = ms * 1e-3
    return dict(workload=w.name, batch=w.batch, seq_len=w.seqlen, nheads=w.nheads, headdim=P,
                ngroups=w.ngroups, d_state=N, us_per_call=round(ms * 1e3, 2),
                elements_per_s=round(w.elements / sec, 1),
                kernel="scan2_mfma_kernel (chunked dual form, 64-step chunks, bf16 MFMA)",
                roofline=dict(bound="hbm", achieved=round(nbytes / sec / 1e9, 1),
                              peak=PEAK_HBM_GBPS, unit="GB/s",
                              frac=round(nbytes / sec / 1e9 / PEAK_HBM_GBPS, 4),
                              traffic=measured_traffic(w.name)),
                mfma=dict(algorithmic_tflops=round(flops / sec / 1e12, 1),
                          executed_tflops=round(flops_exec / sec / 1e12, 1),
                          peak_tflops=PEAK_BF16_TFLOPS,
                          frac_executed=round(flops_exec / sec / 1e12 / PEAK_BF16_TFLOPS, 4)),
                hbm=dict(algorithmic_bytes=nbytes),
                parity_spot_check=dict(ok=ok, max_abs_err=float(err.max())))


def cpu_baseline(args, np, w, p):
    """The fp64 oracle (never tuned) on this host's cores, on the same workload.  Starts from a
    sample of rows and grows it until one run takes >= args.cpu_seconds or covers every row;
    the whole 2.8B layer takes well under that, so it is then repeated to fill the time."""
    import oracle
    threads = max(1, len(os.sched_getaffinity(0)))
    rows_all = w.batch * w.d_inner
    rng = np.random.default_rng(0)
    n = 64
    while True:
        rows = None if n >= rows_all else np.sort(
            rng.choice(rows_all, size=n, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        oracle.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["D"], z=p["z"],
                        delta_bias=p["delta_bias"], rows=rows, nthreads=threads)
        dt = time.perf_counter() - t0
        if dt >= args.cpu_seconds or n >= rows_all:
            break
        n = min(rows_all, max(n * 2, int(n * args.cpu_seconds / max(dt, 1e-3) * 1.05)))
    nrows = rows_all if rows is None else len(rows)
    reps, total = 1, dt
    while total < args.cpu_seconds:
        t0 = time.perf_counter()
        oracle.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["D"], z=p["z"],
                        delta_bias=p["delta_bias"], rows=rows, nthreads=threads)
        total += time.perf_counter() - t0
        reps += 1
    elems = nrows * w.seqlen * reps
    log(f"cpu oracle: {nrows} rows x {w.seqlen} steps x {reps} runs in {total:.1f} s on "
        f"{threads} threads")
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return dict(value=round(elems / total, 1), unit="elements/s", cores=threads, kind="oracle",
                sample=f"{nrows} of {rows_all} (b,d) rows of {w.name}, all {w.seqlen} steps, "
                       f"{reps} run(s), {total:.1f} s wall",
                cpu_model=model)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported (the scan "
              "is measured on one MI355X; a multi-GPU run would split batch rows or channel "
              "blocks across GPUs with no communication inside the scan)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from selective_state_space_36_amd import ops
    from selective_state_space_36_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    ops.lib()

    (w, p, ms_step, ms_kernel, ms_zoh, ms_conv, ms_bwd, train, ok,
     maxerr) = bench_prefill(args, torch, np, ops, wl)
    elems = w.elements
    value = elems / (ms_step * 1e-3)
    nbytes = prefill_bytes(w)
    slots = elems * (w.d_state * SLOTS_PER_UPDATE +
                     (SLOTS_PER_ELEMENT_GATED if w.gate else SLOTS_PER_ELEMENT_PLAIN))
    achieved_slots = slots / (ms_kernel * 1e-3)
    hbm_gbps = nbytes / (ms_kernel * 1e-3) / 1e9
    result = {
        "metric": "selective-scan fwd elements/s (B*L*D) + achieved HBM GB/s; decode step us",
        "value": round(value, 1),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 io, f32 math and state" if w.io_dtype == "bf16" else "f32",
        "data": "synthetic (seeded, Mamba layer-shaped; no weights or datasets)",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen,
                   "d_inner": w.d_inner, "d_state": w.d_state, "gate": "silu(z)",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "alu", "achieved": round(achieved_slots / 1e12, 3),
                     "peak": round(PEAK_VALU_SLOTS / 1e12, 3), "unit": "T VALU-slot/s",
                     "frac": round(achieved_slots / PEAK_VALU_SLOTS, 4),
                     "traffic": measured_traffic(w.name),
                     "kernel": "scan_kernel (prefill output pass)",
                     "kernel_us": round(ms_kernel * 1e3, 2)},
        "hbm": {"algorithmic_bytes": nbytes, "achieved_GBps": round(hbm_gbps, 1),
                "peak_GBps": PEAK_HBM_GBPS, "frac": round(hbm_gbps / PEAK_HBM_GBPS, 4)},
        # transcendentals: one v_exp_f32 per update, and per element 2 for softplus (exp, log)
        # and 2 for silu (exp, rcp); v_exp_f32 issues at half the VALU rate
        "exp": {"per_update": 1,
                "per_element": w.d_state + (4 if w.gate else 2),
                "exp_per_s": round(elems * (w.d_state + (2 if w.gate else 1))
                                   / (ms_kernel * 1e-3), 1),
                "exp_peak_per_s": PEAK_VALU_SLOTS / 2,
                "exp_frac": round(elems * (w.d_state + (2 if w.gate else 1))
                                  / (ms_kernel * 1e-3) / (PEAK_VALU_SLOTS / 2), 4)},
        "zoh_exact": {"kernel_us": round(ms_zoh * 1e3, 2),
                      "elements_per_s": round(elems / (ms_zoh * 1e-3), 1),
                      "note": "same layer with the exact zero-order-hold input term; its extra "
                              "per-update work (a series or (2^y-1)/A, a compare, a select) "
                              "is not in the slot count"},
        "conv_front_end": {"kernel_us": round(ms_conv * 1e3, 2),
                           "elements_per_s": round(elems / (ms_conv * 1e-3), 1),
                           "hbm_bytes_avoided": 2 * elems * (2 if w.io_dtype == "bf16" else 4),
                           "note": "ss_scan_fwd_conv, width-4 causal depthwise conv + SiLU on x "
                                   "fused in; an unfused front end would write u and read it "
                                   "back (hbm_bytes_avoided)"},
        "backward": {"us_per_call": round(ms_bwd * 1e3, 2),
                     "elements_per_s": round(elems / (ms_bwd * 1e-3), 1),
                     "ratio_to_forward": round(ms_bwd / ms_kernel, 2),
                     "note": "ss_scan_bwd (forward pass storing chunk-end states + reverse pass "
                             "recomputing each chunk), all input gradients",
                     "with_saved_states": {
                         "forward_us": round(train["ms_fwd_states"] * 1e3, 2),
                         "backward_us": round(train["ms_bwd_states"] * 1e3, 2),
                         "note": "ss_scan_fwd_states (the forward also writing the 335 MB of "
                                 "chunk-end states) then ss_scan_bwd with SS_FLAG_STATES_GIVEN "
                                 "(no forward pass of its own)"}},
        "parity_spot_check": {"ok": ok, "max_abs_err": maxerr},
    }
    if not args.no_multihead:
        result["multihead"] = bench_multihead(args, torch, np, ops, wl)
    if not args.no_decode:
        result["decode"] = bench_decode(args, torch, np, ops, wl)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, np, w, p)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
