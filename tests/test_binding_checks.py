"""The torch-level binding rejects mismatched buffers before it calls the library (no GPU).

A caller-supplied `out` (or operand) with the wrong shape, dtype, device or layout would
make a kernel write past the end of an allocation or read bytes in the wrong format: the
binding raises ValueError first.  The library's compute entry points are replaced by
functions that fail the test, so a check that lets a bad call through is caught.
"""
import pytest
import torch

from block_scaled_fp4_06_amd import nvfp4 as N


@pytest.fixture(autouse=True)
def no_library_calls(monkeypatch):
    def boom(*a, **k):
        raise AssertionError("the library was called")
    for name in ("nvfp4_quantize", "nvfp4_dequantize", "nvfp4_gemm", "nvfp4_gemm_ws",
                 "nvfp4_transpose_bf16", "mxfp4_quantize", "mxfp4_dequantize", "mxfp4_gemm"):
        monkeypatch.setattr(N, name, boom)
    monkeypatch.setattr(N, "nvfp4_quantize_workspace_bytes", lambda: 1024)
    monkeypatch.setattr(N, "nvfp4_gemm_workspace_bytes", lambda: 2048)


def nv(rows, cols, blocking=N.BLOCK_1x16, device="cpu"):
    s = (rows // 16, cols // 16) if blocking == N.BLOCK_16x16 else (rows, cols // 16)
    return N.NVFP4Tensor(torch.zeros((rows, cols // 2), dtype=torch.uint8, device=device),
                         torch.zeros(s, dtype=torch.uint8, device=device),
                         torch.ones(1, dtype=torch.float32, device=device), rows, cols, blocking)


def mx(rows, cols):
    return N.MXFP4Tensor(torch.zeros((rows, cols // 2), dtype=torch.uint8),
                         torch.zeros((rows, cols // 32), dtype=torch.uint8), rows, cols)


def test_dequantize_out_checks():
    q = nv(32, 64)
    for bad, what in ((torch.empty((32, 64), dtype=torch.float16), "dtype"),
                      (torch.empty((32, 64), dtype=torch.int32), "dtype"),
                      (torch.empty((32, 48), dtype=torch.float32), "shape"),
                      (torch.empty((16, 64), dtype=torch.bfloat16), "shape"),
                      (torch.empty((64, 32), dtype=torch.float32).t(), "row-major"),
                      (torch.empty((32, 128), dtype=torch.float32)[:, ::2], "row-major")):
        with pytest.raises(ValueError, match=what):
            N.dequantize(q, out=bad)
    # a well-formed call on CPU tensors stops at the device check, not in the library
    with pytest.raises(ValueError, match="GPU"):
        N.dequantize(q, out=torch.empty((32, 64), dtype=torch.float32))
    # a wider row stride is a legal layout
    with pytest.raises(ValueError, match="GPU"):
        N.dequantize(q, out=torch.empty((32, 80), dtype=torch.float32)[:, :64])


def test_dequantize_operand_checks():
    q = nv(32, 64)
    q.scales = torch.zeros((32, 2), dtype=torch.uint8)
    with pytest.raises(ValueError, match="scales"):
        N.dequantize(q)
    q = nv(32, 64)
    q.global_dec = torch.ones(1, dtype=torch.float64)
    with pytest.raises(ValueError, match="global_dec"):
        N.dequantize(q)
    q = nv(32, 64)
    q.codes = torch.zeros((32, 64), dtype=torch.uint8)[:, ::2]
    with pytest.raises(ValueError, match="contiguous"):
        N.dequantize(q)


def test_gemm_checks():
    a, b = nv(32, 64), nv(48, 64, N.BLOCK_16x16)
    for bad, what in ((torch.empty((32, 48), dtype=torch.float16), "dtype"),
                      (torch.empty((48, 32), dtype=torch.float32), "shape"),
                      (torch.empty((48, 32), dtype=torch.bfloat16).t(), "row-major")):
        with pytest.raises(ValueError, match=what):
            N.gemm(a, b, out=bad)
    with pytest.raises(ValueError, match="K mismatch"):
        N.gemm(a, nv(48, 32))
    b.scales = torch.zeros((48, 4), dtype=torch.uint8)   # 1x16 layout on a 16x16 operand
    with pytest.raises(ValueError, match="b.scales"):
        N.gemm(a, b)
    b = nv(48, 64, N.BLOCK_16x16)
    with pytest.raises(ValueError, match="workspace"):
        N.gemm(a, b, workspace=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU"):
        N.gemm(a, b, out=torch.empty((32, 48), dtype=torch.float32))


def test_quantize_out_checks():
    x = torch.zeros((32, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="made for"):
        N.quantize(x, out=nv(32, 32))
    with pytest.raises(ValueError, match="made for"):
        N.quantize(x, blocking="16x16", out=nv(32, 64))
    out = nv(32, 64)
    out.codes = torch.zeros((32, 16), dtype=torch.uint8)
    with pytest.raises(ValueError, match="codes"):
        N.quantize(x, out=out)
    out = nv(32, 64, N.BLOCK_16x16)
    with pytest.raises(ValueError, match="with_transpose"):
        N.quantize(x, blocking="16x16", with_transpose=True, out=out)
    out.codes_t = torch.zeros((64, 8), dtype=torch.uint8)
    out.scales_t = torch.zeros((4, 2), dtype=torch.uint8)
    with pytest.raises(ValueError, match="codes_t"):
        N.quantize(x, blocking="16x16", with_transpose=True, out=out)
    with pytest.raises(ValueError, match="workspace"):
        N.quantize(x, workspace=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="workspace"):
        N.quantize(x, workspace=torch.zeros(4096, dtype=torch.int32))
    with pytest.raises(ValueError, match="bf16"):
        N.quantize(torch.zeros((32, 64), dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        N.quantize(x)


def test_mx_and_transpose_checks():
    a, b = mx(32, 64), mx(48, 64)
    with pytest.raises(ValueError, match="dtype"):
        N.mx_gemm(a, b, out=torch.empty((32, 48), dtype=torch.float16))
    with pytest.raises(ValueError, match="shape"):
        N.mx_dequantize(a, out=torch.empty((32, 32), dtype=torch.float32))
    with pytest.raises(ValueError, match="made for"):
        N.mx_quantize(torch.zeros((32, 64), dtype=torch.bfloat16), out=mx(32, 32))
    a.scales = torch.zeros((32, 4), dtype=torch.uint8)
    with pytest.raises(ValueError, match="scales"):
        N.mx_dequantize(a)
    x = torch.zeros((32, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        N.transpose(x, out=torch.empty((32, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="dtype"):
        N.transpose(x, out=torch.empty((64, 32), dtype=torch.float16))
    with pytest.raises(ValueError, match="GPU"):
        N.transpose(x)
