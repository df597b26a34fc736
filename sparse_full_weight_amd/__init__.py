"""Sparse-first fine-tuning hot path for AMD MI355X (gfx950).

The computation lives in ``libsft.so`` (hand-written HIP kernels behind the C
ABI in ``include/sft.h``); ``sparse_full_weight_amd._lib`` is its ctypes
binding and ``sparse_full_weight_amd.synth`` the seeded input generators.
Importing the package loads nothing; the first call into ``_lib`` loads the
library and raises if it has not been built.
"""
__all__ = ["synth", "_lib"]
