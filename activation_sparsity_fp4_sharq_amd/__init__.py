"""SharQ sparse-dense FP4 linear layer for AMD MI355X (gfx950).

The compute path is the HIP library ``libsharq.so`` (kernels + C ABI declared in
``include/sharq.h``); ``sharq`` below is a thin ctypes binding over it.  Importing
this package loads nothing; the library is loaded on the first call and a missing
library is an error (there is no CPU fallback).
"""
from .workloads import MXFP4, NVFP4  # noqa: F401

__all__ = ["MXFP4", "NVFP4"]
