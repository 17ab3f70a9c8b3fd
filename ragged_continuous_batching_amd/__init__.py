"""Ragged continuous-batching attention for AMD Instinct MI355X (gfx950).

The compute path is libcb.so (HIP kernels plus a host step builder) behind the C ABI in
include/cb.h; ``ragged_continuous_batching_amd.cb`` is its ctypes binding, and importing it
fails if the library has not been built (``python -m ragged_continuous_batching_amd.build``).
"""
__all__ = ["cb", "runner", "build"]
