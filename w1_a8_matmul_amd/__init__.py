"""W1.58A8 BitLinear forward on MI355X (gfx950).

The compute path is the C-ABI library ``libbitlinear.so`` (hand-written HIP
kernels, declared in ``include/bitlinear.h``); ``w1_a8_matmul_amd.bitlinear``
is its thin ctypes binding.  ``workloads`` holds the seeded input generators.
Importing the package loads nothing; the binding loads the library on first
use and raises if it is missing.
"""
__all__ = ["bitlinear", "workloads"]
