"""Deja Vu contextually sparse decode layer for AMD MI355X (gfx950).

The compute path is libdejavu.so (hand-written HIP behind a C ABI, see
``include/dejavu.h``); ``contextual_sparsity_amd.dejavu`` is its ctypes binding.
Importing the package loads nothing; the library is loaded on first use and a missing
library is an error, never a fallback.
"""
__all__ = ["dejavu", "synth", "configs", "build"]
