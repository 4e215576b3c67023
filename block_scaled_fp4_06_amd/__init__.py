"""libnvfp4 for AMD MI355X (gfx950): NVFP4 block-scaled FP4 quantize, dequantize, GEMM.

The compute runs in hand-written HIP kernels inside ``libnvfp4.so`` behind a C ABI
(``include/nvfp4.h``); ``block_scaled_fp4_06_amd.nvfp4`` is the thin ctypes binding with
the same names.  Importing this package loads nothing; the library is opened on the
first call and a missing library raises instead of falling back to anything else.
"""
__all__ = ["nvfp4", "workloads"]
