"""Batch-invariant RMSNorm forward/backward for AMD MI355X (gfx950).

The compute path is the HIP library ``csrc/`` builds (C-ABI declared in
``include/rmsnorm_bi.h``); ``binding`` is its thin ctypes binding.  Importing
this package loads nothing: the library is loaded on first use of
``binding``, and a missing library is an error, never a fallback.
"""
__all__ = ["inputs", "layouts"]
