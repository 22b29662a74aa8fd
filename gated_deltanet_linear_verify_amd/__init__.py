"""Gated DeltaNet speculative-verify path for AMD MI355X (gfx950).

The compute lives in ``libgdn.so`` (hand-written HIP kernels behind a C ABI, declared in
``include/gdn.h``).  ``gated_deltanet_linear_verify_amd.gdn`` is the thin ctypes binding;
``workloads`` holds the seeded synthetic inputs.  Importing the package loads nothing.
"""
