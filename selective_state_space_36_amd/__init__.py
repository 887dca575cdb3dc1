"""MI355X-native selective state-space scan (S6): prefill and single-token decode.

The compute path is the C-ABI library ``libssscan.so`` built from ``csrc/`` with hipcc for
gfx950; ``ops`` is a thin ctypes binding over it.  ``workloads`` draws the seeded synthetic
inputs.  Importing this package loads nothing; the library is opened on first use.
"""
