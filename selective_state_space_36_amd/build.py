"""Build libssscan.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libssscan.so")
SOURCES = ["ss_api.hip", "ss_scan_fwd.hip", "ss_state_update.hip"]
ARCH = "gfx950"

# Packed fp32 VALU instructions are disabled (-packed-fp32-ops); the host pass warns that it
# does not know the feature, which is harmless.
FLAGS = [
    "-O3", "-std=c++20", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libssscan.so")
    return exe


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
