"""Focus group-gated sparse attention forward pass on AMD Instinct MI355X (gfx950).

The compute lives in ``libfocus.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/focus.h``); ``group_gated_sparse_amd.focus`` is the thin
ctypes binding. Importing this package loads nothing: the library is opened
on first use and a missing library is an error, never a fallback.
"""
__all__ = ["workloads", "synth", "focus"]
