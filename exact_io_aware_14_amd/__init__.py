"""Exact tiled attention (forward + backward) for AMD MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C-ABI library
``libfa.so`` (declared in ``include/fa.h``); ``exact_io_aware_14_amd.fa`` is the
thin ctypes binding over it.  PyTorch only provides device memory and streams.
"""
__all__ = ["fa", "inputs", "accounting"]
