"""ctypes binding of libnvfp4 (include/nvfp4.h).

Argument marshalling only: every step of quantize, dequantize and the GEMM runs in the
library's HIP kernels.  PyTorch supplies device memory and the current stream.  The
library is loaded from this package directory; if it is missing or cannot be loaded the
call raises -- there is no other implementation to fall back to.

Low-level functions carry the C names (``nvfp4_quantize`` ...) and take raw pointers;
``quantize`` / ``dequantize`` / ``gemm`` wrap them for torch tensors.
"""
from __future__ import annotations

import atexit
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

NVFP4_OK = 0
BLOCK_1x16, BLOCK_16x16 = 0, 1
ROUND_RNE, ROUND_STOCHASTIC = 0, 1
OUT_BF16, OUT_FP32 = 0, 1
_BLOCKING = {"1x16": BLOCK_1x16, "16x16": BLOCK_16x16, 0: 0, 1: 1}
_ROUNDING = {"rne": ROUND_RNE, "sr": ROUND_STOCHASTIC, "stochastic": ROUND_STOCHASTIC, 0: 0, 1: 1}


class QuantParams(ctypes.Structure):
    _fields_ = [("blocking", ctypes.c_int32), ("rounding", ctypes.c_int32),
                ("rht", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("rht_seed", ctypes.c_uint64), ("sr_seed", ctypes.c_uint64),
                ("sr_index_base", ctypes.c_uint64)]


class Operand(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("global_dec", ctypes.c_void_p), ("blocking", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, nvfp4_status_string(status), status))


EXPORTED = ("nvfp4_quantize_workspace_bytes", "nvfp4_quantize", "nvfp4_quantize_noalloc",
            "nvfp4_dequantize",
            "nvfp4_gemm", "nvfp4_gemm_workspace_bytes", "nvfp4_gemm_ws", "nvfp4_transpose_bf16", "mxfp4_quantize", "mxfp4_dequantize",
            "mxfp4_gemm",
            "nvfp4_status_string", "nvfp4_abi_version")

_lib = None


def load(path: str = LIB_PATH):
    """Open libnvfp4.so and declare the C signatures.  Raises if the library is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libnvfp4.so not built (expected at %s); run "
                           "`python -m block_scaled_fp4_06_amd.build`" % path)
    L = ctypes.CDLL(path)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.nvfp4_quantize_workspace_bytes.argtypes = []
    L.nvfp4_quantize_workspace_bytes.restype = ctypes.c_size_t
    L.nvfp4_quantize.argtypes = [P, i64, i64, i64, ctypes.POINTER(QuantParams), P, P, P, P, P,
                                 P, P, ctypes.c_size_t, P]
    L.nvfp4_quantize.restype = ctypes.c_int
    L.nvfp4_quantize_noalloc.argtypes = [P, i64, i64, i64, ctypes.POINTER(QuantParams), P, P,
                                         P, P, P, P, P]
    L.nvfp4_quantize_noalloc.restype = ctypes.c_int
    L.nvfp4_dequantize.argtypes = [P, P, P, i64, i64, i32, P, i64, i32, P]
    L.nvfp4_dequantize.restype = ctypes.c_int
    L.nvfp4_gemm.argtypes = [ctypes.POINTER(Operand), ctypes.POINTER(Operand), i64, i64, i64,
                             P, i64, i32, P]
    L.nvfp4_gemm.restype = ctypes.c_int
    L.nvfp4_gemm_workspace_bytes.argtypes = []
    L.nvfp4_gemm_workspace_bytes.restype = ctypes.c_size_t
    L.nvfp4_gemm_ws.argtypes = [ctypes.POINTER(Operand), ctypes.POINTER(Operand), i64, i64, i64,
                                P, i64, i32, P, ctypes.c_size_t, P]
    L.nvfp4_gemm_ws.restype = ctypes.c_int
    L.nvfp4_transpose_bf16.argtypes = [P, i64, i64, i64, P, i64, P]
    L.nvfp4_transpose_bf16.restype = ctypes.c_int
    L.mxfp4_quantize.argtypes = [P, i64, i64, i64, P, P, P]
    L.mxfp4_quantize.restype = ctypes.c_int
    L.mxfp4_dequantize.argtypes = [P, P, i64, i64, P, i64, i32, P]
    L.mxfp4_dequantize.restype = ctypes.c_int
    L.mxfp4_gemm.argtypes = [P, P, P, P, i64, i64, i64, P, i64, i32, P]
    L.mxfp4_gemm.restype = ctypes.c_int
    L.nvfp4_status_string.argtypes = [ctypes.c_int]
    L.nvfp4_status_string.restype = ctypes.c_char_p
    L.nvfp4_abi_version.argtypes = []
    L.nvfp4_abi_version.restype = ctypes.c_int
    _lib = L
    return L


# ------------------------------------------------------------------ C-named wrappers
def nvfp4_quantize_workspace_bytes() -> int:
    return int(load().nvfp4_quantize_workspace_bytes())


def nvfp4_quantize(x, rows, cols, ld_x, params: QuantParams, codes, scales, global_dec,
                   codes_t, scales_t, dev_status, workspace, workspace_bytes, stream) -> int:
    return int(load().nvfp4_quantize(x, rows, cols, ld_x, ctypes.byref(params), codes, scales,
                                     global_dec, codes_t, scales_t, dev_status, workspace,
                                     workspace_bytes, stream))


def nvfp4_quantize_noalloc(x, rows, cols, ld_x, params: QuantParams, codes, scales,
                           global_dec, codes_t, scales_t, dev_status, stream) -> int:
    return int(load().nvfp4_quantize_noalloc(x, rows, cols, ld_x, ctypes.byref(params), codes,
                                             scales, global_dec, codes_t, scales_t, dev_status,
                                             stream))


def nvfp4_dequantize(codes, scales, global_dec, rows, cols, blocking, y, ld_y, out_dtype,
                     stream) -> int:
    return int(load().nvfp4_dequantize(codes, scales, global_dec, rows, cols, blocking, y,
                                       ld_y, out_dtype, stream))


def nvfp4_gemm(a: Operand, b: Operand, M, N, K, c, ldc, out_dtype, stream) -> int:
    return int(load().nvfp4_gemm(ctypes.byref(a), ctypes.byref(b), M, N, K, c, ldc,
                                 out_dtype, stream))


def nvfp4_gemm_workspace_bytes() -> int:
    return int(load().nvfp4_gemm_workspace_bytes())


def nvfp4_gemm_ws(a: Operand, b: Operand, M, N, K, c, ldc, out_dtype, ws, ws_bytes,
                  stream) -> int:
    return int(load().nvfp4_gemm_ws(ctypes.byref(a), ctypes.byref(b), M, N, K, c, ldc,
                                    out_dtype, ws, ws_bytes, stream))


def nvfp4_transpose_bf16(x, rows, cols, ld_x, y, ld_y, stream) -> int:
    return int(load().nvfp4_transpose_bf16(x, rows, cols, ld_x, y, ld_y, stream))


def mxfp4_quantize(x, rows, cols, ld_x, codes, scales, stream) -> int:
    return int(load().mxfp4_quantize(x, rows, cols, ld_x, codes, scales, stream))


def mxfp4_dequantize(codes, scales, rows, cols, y, ld_y, out_dtype, stream) -> int:
    return int(load().mxfp4_dequantize(codes, scales, rows, cols, y, ld_y, out_dtype, stream))


def mxfp4_gemm(a_codes, a_scales, b_codes, b_scales, M, N, K, c, ldc, out_dtype,
               stream) -> int:
    return int(load().mxfp4_gemm(a_codes, a_scales, b_codes, b_scales, M, N, K, c, ldc,
                                 out_dtype, stream))


def nvfp4_status_string(status: int) -> str:
    return load().nvfp4_status_string(status).decode()


def nvfp4_abi_version() -> int:
    return int(load().nvfp4_abi_version())


# ------------------------------------------------------------------ torch helpers
@dataclass
class NVFP4Tensor:
    """Quantized tensor: codes (rows, cols//2) uint8, scales uint8, global_dec (1,) fp32."""
    codes: "object"
    scales: "object"
    global_dec: "object"
    rows: int
    cols: int
    blocking: int
    codes_t: Optional[object] = None
    scales_t: Optional[object] = None
    status: Optional[object] = None

    def transposed(self) -> "NVFP4Tensor":
        """The W^T operand emitted alongside a 16x16 quantization (same tensor scale)."""
        if self.codes_t is None:
            raise ValueError("quantize(..., with_transpose=True) was not requested")
        return NVFP4Tensor(self.codes_t, self.scales_t, self.global_dec, self.cols, self.rows,
                           self.blocking)


def _stream(stream, device):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _check_buffer(name, t, shape, dtypes, device, row_major=True):
    """Raise ValueError unless tensor t has the given shape, one of `dtypes` and `device`,
    and (row_major) unit column stride with a row stride of at least its width: the layout
    the library writes or reads through the raw pointer."""
    if t is None:
        raise ValueError("%s is missing" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype not in dtypes:
        raise ValueError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if row_major and len(shape) == 2 and shape[0] > 0 and shape[1] > 0:
        if t.stride(1) != 1 or t.stride(0) < shape[1]:
            raise ValueError("%s must be row-major with unit column stride" % name)
    elif not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _require_gpu(device):
    """The last check before a library call: every buffer lives on this GPU device."""
    if device.type != "cuda":
        raise ValueError("tensors must be on a GPU device, not %s" % device)


def _check_workspace(ws, need, device):
    import torch
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor")
    if ws.numel() < need:
        raise ValueError("workspace has %d bytes, needs %d" % (ws.numel(), need))
    if ws.device != device:
        raise ValueError("workspace is on %s, expected %s" % (ws.device, device))


def _check_nvfp4(name, q, device=None):
    """The buffers of an NVFP4Tensor have the documented shapes, dtypes and one device."""
    import torch
    device = q.codes.device if device is None else device
    if q.blocking not in (BLOCK_1x16, BLOCK_16x16):
        raise ValueError("%s.blocking must be 0 (1x16) or 1 (16x16)" % name)
    sshape = (q.rows // 16, q.cols // 16) if q.blocking == BLOCK_16x16 else (q.rows, q.cols // 16)
    u8 = (torch.uint8,)
    _check_buffer(name + ".codes", q.codes, (q.rows, q.cols // 2), u8, device, False)
    _check_buffer(name + ".scales", q.scales, sshape, u8, device, False)
    _check_buffer(name + ".global_dec", q.global_dec, (1,), (torch.float32,), device, False)


def _out_dtypes():
    import torch
    return (torch.float32, torch.bfloat16)


_WORKSPACES = {}
_GEMM_WORKSPACES = {}


def release_workspaces():
    """Wait for the work queued on every device that holds a cached workspace, then drop
    the cached workspaces (one quantize and one GEMM workspace per (device, stream)).  Runs
    at interpreter exit, so the tensors go back to torch while its allocator and the HIP
    runtime are still up and no launch of ours is in flight when the process ends."""
    devices = {k[0] for k in list(_WORKSPACES) + list(_GEMM_WORKSPACES)}
    if devices:
        import torch
        for d in devices:
            try:
                torch.cuda.synchronize(d)
            except RuntimeError:
                pass
    _WORKSPACES.clear()
    _GEMM_WORKSPACES.clear()


atexit.register(release_workspaces)


def new_workspace(device):
    """A quantize workspace: nvfp4_quantize_workspace_bytes() bytes, zero-filled as the
    library requires before first use."""
    import torch
    return torch.zeros(nvfp4_quantize_workspace_bytes(), dtype=torch.uint8, device=device)


def _workspace(dev, stream_handle):
    """One workspace per (device, stream): calls on one stream run in order, so they can
    share it; calls on different streams never do."""
    key = (dev.index, stream_handle)
    ws = _WORKSPACES.get(key)
    if ws is None:
        ws = new_workspace(dev)
        _WORKSPACES[key] = ws
    return ws


def quantize(x, blocking="1x16", rounding="rne", rht=False, rht_seed=0, sr_seed=0,
             sr_index_base=0, with_transpose=False, stream=None, out=None,
             workspace=None) -> NVFP4Tensor:
    """Quantize a 2-D bf16 CUDA tensor (row stride x.stride(0)) to NVFP4.

    workspace: optional uint8 CUDA tensor from new_workspace(), used by one stream at a
    time; by default one cached workspace per (device, stream) is used."""
    import torch
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    rows, cols = x.shape
    blk = _BLOCKING[blocking]
    dev = x.device
    if out is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        sshape = (rows // 16, cols // 16) if blk == BLOCK_16x16 else (rows, cols // 16)
        scales = torch.empty(sshape, dtype=torch.uint8, device=dev)
        g = torch.empty(1, dtype=torch.float32, device=dev)
        st = torch.empty(4, dtype=torch.int32, device=dev)
        ct = st_ = None
        if with_transpose:
            ct = torch.empty((cols, rows // 2), dtype=torch.uint8, device=dev)
            st_ = torch.empty((cols // 16, rows // 16), dtype=torch.uint8, device=dev)
        out = NVFP4Tensor(codes, scales, g, rows, cols, blk, ct, st_, st)
    else:
        if (out.rows, out.cols, out.blocking) != (rows, cols, blk):
            raise ValueError("out was made for a %dx%d tensor with blocking %d" %
                             (out.rows, out.cols, out.blocking))
        _check_nvfp4("out", out, dev)
        if with_transpose != (out.codes_t is not None) or (out.codes_t is None) != (out.scales_t is None):
            raise ValueError("out.codes_t/scales_t must be given exactly when with_transpose")
        if out.codes_t is not None:
            _check_buffer("out.codes_t", out.codes_t, (cols, rows // 2), (torch.uint8,), dev, False)
            _check_buffer("out.scales_t", out.scales_t, (cols // 16, rows // 16), (torch.uint8,),
                          dev, False)
        if out.status is not None:
            _check_buffer("out.status", out.status, tuple(out.status.shape), (torch.int32,), dev,
                          False)
    if workspace is not None:
        _check_workspace(workspace, nvfp4_quantize_workspace_bytes(), dev)
    _require_gpu(dev)
    sh = _stream(stream, dev)
    ws = workspace if workspace is not None else _workspace(dev, sh.value)
    prm = QuantParams(blk, _ROUNDING[rounding], 1 if rht else 0, 0, rht_seed, sr_seed,
                      sr_index_base)
    rc = nvfp4_quantize(_ptr(x), rows, cols, x.stride(0), prm, _ptr(out.codes),
                        _ptr(out.scales), _ptr(out.global_dec), _ptr(out.codes_t),
                        _ptr(out.scales_t), _ptr(out.status), _ptr(ws), ws.numel(), sh)
    if rc != NVFP4_OK:
        raise NVFP4Error(rc, "nvfp4_quantize")
    return out


def dequantize(q: NVFP4Tensor, out_dtype=None, stream=None, out=None):
    """x = e2m1(code) * e4m3(scale) * global as a (rows, cols) float32 or bf16 tensor; `out`
    (optional) must have that shape and dtype, unit column stride, on the codes' device."""
    import torch
    _check_nvfp4("q", q)
    if out is None:
        out = torch.empty((q.rows, q.cols), dtype=out_dtype or torch.bfloat16,
                          device=q.codes.device)
    _check_buffer("out", out, (q.rows, q.cols), _out_dtypes(), q.codes.device)
    _require_gpu(q.codes.device)
    od = OUT_FP32 if out.dtype == torch.float32 else OUT_BF16
    rc = nvfp4_dequantize(_ptr(q.codes), _ptr(q.scales), _ptr(q.global_dec), q.rows, q.cols,
                          q.blocking, _ptr(out), out.stride(0), od,
                          _stream(stream, q.codes.device))
    if rc != NVFP4_OK:
        raise NVFP4Error(rc, "nvfp4_dequantize")
    return out


def new_gemm_workspace(device):
    """A GEMM workspace: nvfp4_gemm_workspace_bytes() bytes, zero-filled as the library
    requires before first use."""
    import torch
    return torch.zeros(nvfp4_gemm_workspace_bytes(), dtype=torch.uint8, device=device)


def gemm(a: NVFP4Tensor, b: NVFP4Tensor, out_dtype=None, stream=None, out=None,
         workspace=None, split_tail=True):
    """C = A . B^T with A (M x K) and B (N x K) NVFP4 operands.

    split_tail: run nvfp4_gemm_ws, which splits the tiles of a last, partial round along K
    (workspace: optional tensor from new_gemm_workspace(), used by one stream at a time; by
    default one cached workspace per (device, stream)); False runs nvfp4_gemm."""
    import torch
    if a.cols != b.cols:
        raise ValueError("K mismatch: %d vs %d" % (a.cols, b.cols))
    dev = a.codes.device
    _check_nvfp4("a", a, dev)
    _check_nvfp4("b", b, dev)
    if out is None:
        out = torch.empty((a.rows, b.rows), dtype=out_dtype or torch.bfloat16, device=dev)
    _check_buffer("out", out, (a.rows, b.rows), _out_dtypes(), dev)
    if split_tail and workspace is not None:
        _check_workspace(workspace, nvfp4_gemm_workspace_bytes(), dev)
    _require_gpu(dev)
    od = OUT_FP32 if out.dtype == torch.float32 else OUT_BF16
    oa = Operand(a.codes.data_ptr(), a.scales.data_ptr(), a.global_dec.data_ptr(), a.blocking, 0)
    ob = Operand(b.codes.data_ptr(), b.scales.data_ptr(), b.global_dec.data_ptr(), b.blocking, 0)
    sh = _stream(stream, dev)
    if split_tail:
        ws = workspace
        if ws is None:
            key = (dev.index, sh.value)
            ws = _GEMM_WORKSPACES.get(key)
            if ws is None:
                ws = _GEMM_WORKSPACES[key] = new_gemm_workspace(dev)
        rc = nvfp4_gemm_ws(oa, ob, a.rows, b.rows, a.cols, _ptr(out), out.stride(0), od,
                           _ptr(ws), ws.numel(), sh)
        name = "nvfp4_gemm_ws"
    else:
        rc = nvfp4_gemm(oa, ob, a.rows, b.rows, a.cols, _ptr(out), out.stride(0), od, sh)
        name = "nvfp4_gemm"
    if rc != NVFP4_OK:
        raise NVFP4Error(rc, name)
    return out


def transpose(x, stream=None, out=None):
    """x^T of a 2-D bf16 CUDA tensor (unit column stride), contiguous."""
    import torch
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    rows, cols = x.shape
    if out is None:
        out = torch.empty((cols, rows), dtype=torch.bfloat16, device=x.device)
    _check_buffer("out", out, (cols, rows), (torch.bfloat16,), x.device)
    _require_gpu(x.device)
    rc = nvfp4_transpose_bf16(_ptr(x), rows, cols, x.stride(0), _ptr(out), out.stride(0),
                              _stream(stream, x.device))
    if rc != NVFP4_OK:
        raise NVFP4Error(rc, "nvfp4_transpose_bf16")
    return out


# ------------------------------------------------------------------ MXFP4
@dataclass
class MXFP4Tensor:
    """MXFP4 tensor: codes (rows, cols//2) uint8, scales (rows, cols//32) uint8 (E8M0)."""
    codes: "object"
    scales: "object"
    rows: int
    cols: int


def _check_mx(name, q, device=None):
    import torch
    device = q.codes.device if device is None else device
    _check_buffer(name + ".codes", q.codes, (q.rows, q.cols // 2), (torch.uint8,), device, False)
    _check_buffer(name + ".scales", q.scales, (q.rows, q.cols // 32), (torch.uint8,), device,
                  False)


def mx_quantize(x, stream=None, out=None) -> MXFP4Tensor:
    """Quantize a 2-D bf16 CUDA tensor (row stride x.stride(0)) to MXFP4."""
    import torch
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    rows, cols = x.shape
    dev = x.device
    if out is None:
        out = MXFP4Tensor(torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev),
                          torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev),
                          rows, cols)
    else:
        if (out.rows, out.cols) != (rows, cols):
            raise ValueError("out was made for a %dx%d tensor" % (out.rows, out.cols))
        _check_mx("out", out, dev)
    _require_gpu(dev)
    rc = mxfp4_quantize(_ptr(x), rows, cols, x.stride(0), _ptr(out.codes), _ptr(out.scales),
                        _stream(stream, dev))
    if rc != NVFP4_OK:
        raise NVFP4Error(rc, "mxfp4_quantize")
    return out


def mx_dequantize(q: MXFP4Tensor, out_dtype=None, stream=None, out=None):
    import torch
    _check_mx("q", q)
    if out is None:
        out = torch.empty((q.rows, q.cols), dtype=out_dtype or torch.bfloat16,
                          device=q.codes.device)
    _check_buffer("out", out, (q.rows, q.cols), _out_dtypes(), q.codes.device)
    _require_gpu(q.codes.device)
    od = OUT_FP32 if out.dtype == torch.float32 else OUT_BF16
    rc = mxfp4_dequantize(_ptr(q.codes), _ptr(q.scales), q.rows, q.cols, _ptr(out),
                          out.stride(0), od, _stream(stream, q.codes.device))
    if rc != NVFP4_OK:
        raise NVFP4Error(rc, "mxfp4_dequantize")
    return out


def mx_gemm(a: MXFP4Tensor, b: MXFP4Tensor, out_dtype=None, stream=None, out=None):
    """C = A . B^T with A (M x K) and B (N x K) MXFP4 operands."""
    import torch
    if a.cols != b.cols:
        raise ValueError("K mismatch: %d vs %d" % (a.cols, b.cols))
    dev = a.codes.device
    _check_mx("a", a, dev)
    _check_mx("b", b, dev)
    if out is None:
        out = torch.empty((a.rows, b.rows), dtype=out_dtype or torch.bfloat16, device=dev)
    _check_buffer("out", out, (a.rows, b.rows), _out_dtypes(), dev)
    _require_gpu(dev)
    od = OUT_FP32 if out.dtype == torch.float32 else OUT_BF16
    rc = mxfp4_gemm(_ptr(a.codes), _ptr(a.scales), _ptr(b.codes), _ptr(b.scales), a.rows,
                    b.rows, a.cols, _ptr(out), out.stride(0), od,
                    _stream(stream, a.codes.device))
    if rc != NVFP4_OK:
        raise NVFP4Error(rc, "mxfp4_gemm")
    return out
