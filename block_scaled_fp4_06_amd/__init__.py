"""libnvfp4 for AMD MI355X (gfx950): NVFP4 block-scaled FP4 quantize, dequantize, GEMM.

The compute runs in hand-written HIP kernels inside ``libnvfp4.so`` behind a C ABI
(``include/nvfp4.h``): NVFP4 quantize (1x16 or 16x16 blocks, optional 16-point random
Hadamard transform, nearest-even or stochastic rounding, W^T from the same read),
dequantize and GEMM; the MXFP4 variant (quantize, dequantize, GEMM on the scaled FP4
matrix instructions); and a bf16 transpose.  ``block_scaled_fp4_06_amd.nvfp4`` is the thin
ctypes binding with the same names; ``block_scaled_fp4_06_amd.linear`` sequences those calls
into a linear layer's forward and backward products.  Importing this package loads nothing;
the library is opened on the first call and a missing library raises instead of falling
back to anything else.
"""
__all__ = ["nvfp4", "linear", "workloads"]
