"""FP4 block-scaled quantization and GEMM for MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``libfp4_mi355x.so``, declared in ``include/fp4.h``).  ``api`` is a thin
ctypes binding over it that takes torch device tensors for memory and the
current torch stream; importing this package does not load the library, the
first call does, and it raises if the library is missing.
"""
__all__ = ["api", "inputs"]
