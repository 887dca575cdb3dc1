"""The allocation-free prefill (ss_scan_fwd_noalloc) through the C ABI: on two calls in a row,
the second with a smaller input, its outputs equal ss_scan_fwd's bit for bit (same kernels, same
automatic time split, carries in the library's static scratch instead of a workspace) and match
the fp64 oracle within the stated bounds."""
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
    ops.lib()  # raises if the HIP library is missing: no silent fallback
    yield


def _case(batch, seqlen, d_inner, seed):
    from selective_state_space_36_amd import ops
    w = wl.WORKLOADS[3]
    p = wl.make_prefill(w, batch=batch, seqlen=seqlen, d_inner=d_inner, seed=seed)
    h0 = np.random.default_rng(seed).standard_normal((batch, d_inner, w.d_state)).astype(np.float32)
    g = {k: dev(v) for k, v in p.items()}
    nbytes = ops.workspace_bytes(batch, seqlen, d_inner, w.d_state, torch.bfloat16)
    print(f"  noalloc case: batch={batch} seqlen={seqlen} d_inner={d_inner} (time-split "
          f"workspace {nbytes} bytes)", flush=True)
    return p, h0, g, nbytes


def test_noalloc_matches_workspace_entry_point_twice():
    from selective_state_space_36_amd import ops
    cases = [(1, 20000, 48, 3), (1, 6000, 32, 4), (2, 700, 64, 5)]
    for i, (batch, seqlen, d_inner, seed) in enumerate(cases):
        p, h0, g, nbytes = _case(batch, seqlen, d_inner, seed)
        if i < 2:
            assert nbytes > 0, "the case is meant to take the time split"
        args = (g["u"], g["delta"], g["A"], g["B"], g["C"])
        kw = dict(D=g["D"], z=g["z"], delta_bias=g["delta_bias"], h0=dev(h0))
        out_n = torch.empty_like(g["u"])
        hl_n = torch.empty((batch, d_inner, 16), dtype=torch.float32, device="cuda")
        ops.scan_fwd_noalloc(*args, **kw, out=out_n, h_last=hl_n)
        out_w, hl_w = ops.scan_fwd(*args, **kw, return_last_state=True)
        torch.cuda.synchronize()
        assert torch.equal(out_n.view(torch.int16), out_w.view(torch.int16)), f"case {i}: out"
        assert torch.equal(hl_n, hl_w), f"case {i}: h_last"
        ref, ref_h = oracle.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["D"],
                                     z=p["z"], delta_bias=p["delta_bias"],
                                     h0=h0.astype(np.float64))
        check_close(host(out_n), ref, TOL["bf16"], f"case {i} out")
        check_close(host(hl_n), ref_h, 1e-3, f"case {i} h_last")
