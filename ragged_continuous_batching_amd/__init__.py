"""Ragged continuous-batching attention for AMD Instinct MI355X (gfx950).

The compute path is libcb.so (HIP kernels plus a host step builder) behind the C ABI in
include/cb.h; ``cb`` is its ctypes binding. Importing the package fails if the library has
not been built (``python -m ragged_continuous_batching_amd.build``).
"""
from . import cb  # noqa: F401

__all__ = ["cb"]
