"""NVFP4 linear layer Y = X W: forward and backward products on libnvfp4's kernels.

The three matrix products of a linear layer in training, each on NVFP4 operands (NVIDIA
developer blog zh-cn "NVFP4 trains with precision of 16-bit ...", section "用于预训练的
NVFP4 量化配方", bullets 1-5; prism.simon-ai.net article 7890, sections
"训练稳定性与敏感层保护策略" and "应对异常值与舍入误差的技术手段"):

  Fprop  Y  = X W      X: 1x16 nearest-even;   W^T: from W's 16x16 quantization
  Dgrad  dX = dY W^T   dY: 1x16 stochastic;     W: the same 16x16 quantization
  Wgrad  dW = X^T dY   X^T, dY^T: 1x16 along the token dimension M, both with the random
                       Hadamard transform (one seed), dY^T with stochastic rounding

One 16x16 quantization of W serves both weight products: its codes and their transpose
come from one read, and they agree exactly, which is why weights take 16x16 blocks.  The
transform sits on the Wgrad inputs, which are quantized afresh along M; the weight's one
quantization could not carry a transform along K and along N at once.  Dgrad and Wgrad
draw their stochastic rounding with sr_seed and sr_seed + 1.

This module only sequences library calls (quantize, transpose, GEMM); every arithmetic
step runs in the HIP kernels.  M, K and N must be multiples of 16 (the quantizer's unit);
a call that breaks this raises NVFP4Error from the first quantization.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import nvfp4 as N

DEFAULT_RHT_SEED = 0x5248


@dataclass
class LinearContext:
    """What the backward pass keeps from the forward pass."""
    x: "object"            # bf16 input (M, K), for Wgrad
    qw: N.NVFP4Tensor      # 16x16 quantization of W (K, N) with its transpose
    rht_seed: int
    sr_seed: int


def linear_forward(x, w, rht_seed: int = DEFAULT_RHT_SEED, sr_seed: int = 0, out_dtype=None,
                   stream=None):
    """Y = X W for bf16 x (M, K) and w (K, N); returns (y, ctx)."""
    qx = N.quantize(x, blocking="1x16", rounding="rne", stream=stream)
    qw = N.quantize(w, blocking="16x16", rounding="rne", with_transpose=True, stream=stream)
    y = N.gemm(qx, qw.transposed(), out_dtype=out_dtype, stream=stream)
    return y, LinearContext(x, qw, rht_seed, sr_seed)


def linear_backward(dy, ctx: LinearContext, dx_dtype=None, dw_dtype=None, stream=None):
    """(dX, dW) for the bf16 output gradient dy (M, N)."""
    qdy = N.quantize(dy, blocking="1x16", rounding="sr", sr_seed=ctx.sr_seed, stream=stream)
    dx = N.gemm(qdy, ctx.qw, out_dtype=dx_dtype, stream=stream)
    xt = N.transpose(ctx.x, stream=stream)
    dyt = N.transpose(dy, stream=stream)
    qxt = N.quantize(xt, blocking="1x16", rounding="rne", rht=True, rht_seed=ctx.rht_seed,
                     stream=stream)
    qdyt = N.quantize(dyt, blocking="1x16", rounding="sr", rht=True, rht_seed=ctx.rht_seed,
                      sr_seed=ctx.sr_seed + 1, stream=stream)
    dw = N.gemm(qxt, qdyt, out_dtype=dw_dtype, stream=stream)
    return dx, dw


_AUTOGRAD_FN = None


def autograd_linear():
    """A torch.autograd.Function running the layer's three products on NVFP4 operands
    (bf16 in and out).  Built once, on first use, so that importing the package needs no
    torch."""
    global _AUTOGRAD_FN
    if _AUTOGRAD_FN is not None:
        return _AUTOGRAD_FN
    import torch

    class NVFP4LinearFn(torch.autograd.Function):
        @staticmethod
        def forward(fctx, x, w, rht_seed, sr_seed):
            y, ctx = linear_forward(x.contiguous(), w.contiguous(), rht_seed, sr_seed)
            fctx.lin = ctx
            return y

        @staticmethod
        def backward(fctx, dy):
            dx, dw = linear_backward(dy.contiguous(), fctx.lin, dw_dtype=torch.bfloat16)
            return dx, dw, None, None

    _AUTOGRAD_FN = NVFP4LinearFn
    return NVFP4LinearFn
