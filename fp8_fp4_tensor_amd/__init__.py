"""FP8/FP4 tensor quantization for AMD MI355X (CDNA4, gfx950).

The library itself is libfq.so, a C-ABI shared library of hand-written HIP
kernels (include/fq.h). This package holds its sources (csrc/), the build
step and a thin ctypes binding (`fp8_fp4_tensor_amd.fq`) that passes torch
device pointers and the current HIP stream through to the C entry points.
Importing the package loads nothing; the binding loads libfq.so on first use
and raises if it is missing.
"""
__all__ = ["fq", "workloads"]
