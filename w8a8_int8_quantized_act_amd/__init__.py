"""W8A8 INT8 CausalConv3d for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libqvae.so`` built from ``csrc/``
(hand-written HIP kernels); ``ops`` is its thin ctypes binding.  The library is
loaded on first use, and every call fails loudly when it is missing.
"""
__all__ = ["ops", "workloads"]
