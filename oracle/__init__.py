"""CPU oracle for NVFP4 block-scaled FP4 quantization -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it, and the two
share no code: the arithmetic lives in ``nvfp4_oracle.c`` (plain C, built with gcc,
``-ffp-contract=off``, no fast-math) and this module only marshals numpy arrays.

Functions and the passages they follow (the pages state the method in words):
  * ``quantize`` / ``dequantize`` -- NVIDIA developer blog (zh-cn) "NVFP4 trains with
    precision of 16-bit ...", section "用于预训练的 NVFP4 量化配方", bullets 1-5; the
    prism.simon-ai.net article 7890, sections "MVFP4格式的核心架构革新" (FP32 tensor
    scale over E4M3 block scales), "训练稳定性与敏感层保护策略" (16x16 weight blocks)
    and "应对异常值与舍入误差的技术手段" (random Hadamard transform, stochastic rounding).
  * ``mx_quantize`` / ``mx_block_values_f64`` / ``mx_gemm_reference`` -- MXFP4, the
    32-element power-of-two-scale format the prism article (section "MVFP4与MXFP4") and
    10100.com (section 二(一)) set NVFP4 against; the scale rule is the OCP Microscaling
    Formats v1.0 one (a reading: the pages give none).
  * ``gemm_reference`` -- the linear-layer product the recipe exists for (blog, same
    section, Figure 1 paragraph): the binary64 product of the exactly dequantized
    operands, computed with numpy's matmul (BLAS dgemm) as the one library step.

Parity status: every function is pinned by the ``-m "not gpu"`` tests against facts
the pages or the mathematics fix (value sets, the 6 x 100 = 600 example, the
0.3 -> 30 % example, norm preservation, library casts/transforms, brute force).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liborc_nvfp4.so")

BLOCK_1x16 = 0
BLOCK_16x16 = 1
ROUND_RNE = 0
ROUND_SR = 1
E4M3_MAX = 448.0
E2M1_MAX = 6.0


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liborc_nvfp4.so``."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.check_call(cmd, cwd=_HERE)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Params(ctypes.Structure):
    _fields_ = [("blocking", ctypes.c_int32), ("rounding", ctypes.c_int32),
                ("rht", ctypes.c_int32), ("pad_", ctypes.c_int32),
                ("rht_seed", ctypes.c_uint64), ("sr_seed", ctypes.c_uint64),
                ("sr_index_base", ctypes.c_uint64)]


_lib = None


def declare(L):
    """Declare the C signatures on a loaded oracle library ``L`` (ctypes.CDLL)."""
    P = ctypes.c_void_p
    i64, u64, u8, u16 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint8, ctypes.c_uint16
    L.orc_e2m1_decode.argtypes = [u8]
    L.orc_e2m1_decode.restype = ctypes.c_float
    L.orc_e2m1_encode_rn.argtypes = [ctypes.c_float]
    L.orc_e2m1_encode_rn.restype = u8
    L.orc_e2m1_encode_sr.argtypes = [ctypes.c_float, u16]
    L.orc_e2m1_encode_sr.restype = u8
    L.orc_e4m3_decode.argtypes = [u8]
    L.orc_e4m3_decode.restype = ctypes.c_float
    L.orc_e4m3_encode.argtypes = [ctypes.c_float]
    L.orc_e4m3_encode.restype = u8
    L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    L.orc_f32_to_bf16.restype = u16
    L.orc_f32_to_bf16_array.argtypes = [P, i64, P]
    L.orc_quantize.argtypes = [P, i64, i64, i64, ctypes.POINTER(_Params), P, P, P, P]
    L.orc_quantize.restype = ctypes.c_int
    L.orc_dequantize.argtypes = [P, P, ctypes.c_float, i64, i64, ctypes.c_int, P]
    L.orc_dequantize.restype = ctypes.c_int
    L.orc_dequantize_bf16.argtypes = [P, P, ctypes.c_float, i64, i64, ctypes.c_int, P]
    L.orc_dequantize_bf16.restype = ctypes.c_int
    L.orc_block_values_f64.argtypes = [P, P, i64, i64, ctypes.c_int, P]
    L.orc_block_values_f64.restype = ctypes.c_int
    L.orc_e4m3_encode_array.argtypes = [P, i64, P]
    L.orc_e2m1_encode_rn_array.argtypes = [P, i64, P]
    L.orc_e2m1_encode_sr_array.argtypes = [P, P, i64, P]
    L.orc_philox_array.argtypes = [P, P, i64, P]
    L.orc_sr_bits_array.argtypes = [u64, u64, i64, P]
    L.orc_rht16_rows.argtypes = [P, i64, u64, P]
    L.orc_rht_signs.argtypes = [u64, P]
    L.orc_rht16_rows_signs.argtypes = [P, i64, P, P]
    L.orc_abi_version.restype = ctypes.c_int
    L.orc_mx_scale.argtypes = [ctypes.c_float]
    L.orc_mx_scale.restype = ctypes.c_uint8
    L.orc_mx_quantize.argtypes = [P, i64, i64, i64, P, P, P]
    L.orc_mx_quantize.restype = ctypes.c_int
    L.orc_mx_block_values_f64.argtypes = [P, P, i64, i64, P]
    L.orc_mx_block_values_f64.restype = ctypes.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        _lib = declare(ctypes.CDLL(_LIB_PATH))
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- codecs
def e2m1_decode(codes) -> np.ndarray:
    L = lib()
    c = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([L.orc_e2m1_decode(int(v)) for v in c], dtype=np.float32)


def e2m1_encode_rn(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().orc_e2m1_encode_rn_array(_p(v), v.size, _p(out))
    return out


def e2m1_encode_sr(v: np.ndarray, k: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    k = np.ascontiguousarray(np.broadcast_to(k, v.shape), dtype=np.uint16)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().orc_e2m1_encode_sr_array(_p(v), _p(k), v.size, _p(out))
    return out


def e4m3_decode(codes) -> np.ndarray:
    L = lib()
    c = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([L.orc_e4m3_decode(int(v)) for v in c], dtype=np.float32)


def e4m3_encode(s: np.ndarray) -> np.ndarray:
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.empty(s.shape, dtype=np.uint8)
    lib().orc_e4m3_encode_array(_p(s), s.size, _p(out))
    return out


def philox4x32_10(ctr: np.ndarray, key: np.ndarray) -> np.ndarray:
    """ctr: (n, 4) uint32, key: (n, 2) uint32 -> (n, 4) uint32."""
    ctr = np.ascontiguousarray(ctr, dtype=np.uint32).reshape(-1, 4)
    key = np.ascontiguousarray(np.broadcast_to(key, (ctr.shape[0], 2)), dtype=np.uint32)
    out = np.empty_like(ctr)
    lib().orc_philox_array(_p(ctr), _p(key), ctr.shape[0], _p(out))
    return out


def sr_bits(seed: int, first: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    lib().orc_sr_bits_array(seed, first, n, _p(out))
    return out


def rht_signs(seed: int) -> np.ndarray:
    d = np.empty(16, dtype=np.float32)
    lib().orc_rht_signs(seed, _p(d))
    return d


def rht16(x: np.ndarray, seed: int) -> np.ndarray:
    """Random Hadamard transform of every consecutive 16-element group of x (fp32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.size % 16 == 0
    y = np.empty_like(x)
    lib().orc_rht16_rows(_p(x), x.size // 16, seed, _p(y))
    return y


def rht16_with_signs(x: np.ndarray, d: np.ndarray) -> np.ndarray:
    """The same butterfly with an explicit +-1 sign vector d (16 values)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    d = np.ascontiguousarray(d, dtype=np.float32)
    assert x.size % 16 == 0 and d.size == 16
    y = np.empty_like(x)
    lib().orc_rht16_rows_signs(_p(x), x.size // 16, _p(d), _p(y))
    return y


def f32_to_bf16(f: np.ndarray, L=None) -> np.ndarray:
    """bf16 bit patterns of binary32 values, nearest-even (``orc_f32_to_bf16``)."""
    f = np.ascontiguousarray(f, dtype=np.float32).ravel()
    out = np.empty(f.shape, dtype=np.uint16)
    (L or lib()).orc_f32_to_bf16_array(_p(f), f.size, _p(out))
    return out


# ---------------------------------------------------------------- quantize
class QuantizeError(RuntimeError):
    pass


def quantize(x_bf16: np.ndarray, *, blocking: int = BLOCK_1x16, rounding: int = ROUND_RNE,
             rht: bool = False, rht_seed: int = 0, sr_seed: int = 0,
             sr_index_base: int = 0):
    """Quantize a (rows, cols) bf16 tensor given as uint16 bit patterns.

    Returns (codes uint8 (rows, cols//2), scales uint8, global_dec float32, status int).
    """
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    if blocking == BLOCK_16x16:
        scales = np.zeros((rows // 16, cols // 16), dtype=np.uint8)
    else:
        scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    g = np.zeros(1, dtype=np.float32)
    st = np.zeros(1, dtype=np.uint32)
    prm = _Params(blocking, rounding, 1 if rht else 0, 0, rht_seed, sr_seed, sr_index_base)
    rc = lib().orc_quantize(_p(x), rows, cols, cols, ctypes.byref(prm), _p(codes),
                            _p(scales), _p(g), _p(st))
    if rc < 0:
        raise QuantizeError("oracle rejected the arguments (code %d)" % rc)
    return codes, scales, np.float32(g[0]), int(st[0])


def dequantize(codes: np.ndarray, scales: np.ndarray, global_dec, rows: int, cols: int,
               blocking: int = BLOCK_1x16, L=None) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    y = np.empty((rows, cols), dtype=np.float32)
    rc = (L or lib()).orc_dequantize(_p(codes), _p(scales), float(np.float32(global_dec)), rows,
                              cols, blocking, _p(y))
    if rc != 0:
        raise QuantizeError("bad shape")
    return y


def dequantize_bf16(codes, scales, global_dec, rows, cols, blocking=BLOCK_1x16, L=None):
    """Dequantize to bf16 (uint16 bit patterns): each binary32 value of ``dequantize``
    rounded to nearest-even by the oracle's one bf16 conversion, ``orc_f32_to_bf16``.
    ``L``: another build of the oracle library (tests load planted variants)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    y = np.empty((rows, cols), dtype=np.uint16)
    rc = (L or lib()).orc_dequantize_bf16(_p(codes), _p(scales), float(np.float32(global_dec)),
                                          rows, cols, blocking, _p(y))
    if rc != 0:
        raise QuantizeError("bad shape")
    return y


def block_values_f64(codes, scales, rows, cols, blocking=BLOCK_1x16) -> np.ndarray:
    """Exact e2m1(q) * e4m3(scale) in binary64 (tensor scale not applied)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty((rows, cols), dtype=np.float64)
    rc = lib().orc_block_values_f64(_p(codes), _p(scales), rows, cols, blocking, _p(out))
    if rc != 0:
        raise QuantizeError("bad shape")
    return out


def mx_quantize(x_bf16: np.ndarray):
    """MXFP4 quantize of a (rows, cols) bf16 tensor, cols % 32 == 0.

    Returns (codes uint8 (rows, cols//2), scales uint8 E8M0 (rows, cols//32), status)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 32), dtype=np.uint8)
    st = np.zeros(1, dtype=np.uint32)
    rc = lib().orc_mx_quantize(_p(x), rows, cols, cols, _p(codes), _p(scales), _p(st))
    if rc < 0:
        raise QuantizeError("oracle rejected the arguments (code %d)" % rc)
    return codes, scales, int(st[0])


def mx_scale(amax: float) -> int:
    return int(lib().orc_mx_scale(float(amax)))


def mx_block_values_f64(codes, scales, rows, cols) -> np.ndarray:
    """Exact e2m1(q) * 2^(scale - 127) in binary64."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty((rows, cols), dtype=np.float64)
    if lib().orc_mx_block_values_f64(_p(codes), _p(scales), rows, cols, _p(out)) != 0:
        raise QuantizeError("bad shape")
    return out


def mx_gemm_reference(a, b, row_slice=None) -> np.ndarray:
    """binary64 C = A . B^T for MXFP4 operands given as (codes, scales, rows, cols)."""
    qa = mx_block_values_f64(*a)
    if row_slice is not None:
        qa = qa[row_slice]
    return np.matmul(qa, mx_block_values_f64(*b).T)


def gemm_reference(a, b, row_slice=None) -> np.ndarray:
    """binary64 reference of C = A_deq . B_deq^T for NVFP4 operands.

    ``a`` and ``b`` are (codes, scales, global_dec, rows, cols, blocking) tuples; B is
    given as N x K (K contiguous), i.e. the transposed weight.  C[m, n] =
    s_A * s_B * sum_k (e2m1 * sbd)_A[m, k] * (e2m1 * sbd)_B[n, k]; the per-element
    products are exact in binary64 and numpy's matmul does the sum.
    ``row_slice`` restricts the rows of A (for a bounded sample of a large product).
    """
    ca, sa, ga, ma, ka, bla = a
    cb, sb, gb, nb, kb, blb = b
    assert ka == kb
    qa = block_values_f64(ca, sa, ma, ka, bla)
    if row_slice is not None:
        qa = qa[row_slice]
    qb = block_values_f64(cb, sb, nb, kb, blb)
    c = np.matmul(qa, qb.T)
    c *= float(np.float32(ga)) * float(np.float32(gb))
    return c


def gemm_reference_chunks(a, b, chunk, with_abs=False):
    """``gemm_reference`` in row chunks: yields (r0, r1, C[r0:r1]) and, with ``with_abs``,
    also s_A s_B |A_deq| |B_deq|^T for those rows (the scale of the fp32 summation error).
    The block values are formed once; each chunk is one binary64 matmul (BLAS dgemm)."""
    ca, sa, ga, ma, ka, bla = a
    cb, sb, gb, nb, kb, blb = b
    assert ka == kb
    qa = block_values_f64(ca, sa, ma, ka, bla)
    qbt = np.ascontiguousarray(block_values_f64(cb, sb, nb, kb, blb).T)
    absbt = np.abs(qbt) if with_abs else None
    g = float(np.float32(ga)) * float(np.float32(gb))
    for r0 in range(0, ma, chunk):
        r1 = min(ma, r0 + chunk)
        c = np.matmul(qa[r0:r1], qbt)
        c *= g
        if with_abs:
            yield r0, r1, c, np.matmul(np.abs(qa[r0:r1]), absbt) * abs(g)
        else:
            yield r0, r1, c


# ------------------------------------------------------------------ linear layer
# The three products of a linear layer Y = X W in training, each on quantized operands:
# Fprop Y = X W, Dgrad dX = dY W^T, Wgrad dW = X^T dY (blog, recipe section: the matrix
# products of linear layers are what FP4 accelerates, bullets 1-5 name the quantization
# steps; prism article, training-stability section: the forward pass uses W and the
# backward pass W^T, so weights take 16x16 blocks; outliers section: random Hadamard
# transform, stochastic rounding of gradients).  Readings where the pages leave a choice:
#   * X: 1x16 blocks, nearest-even; W: 16x16 blocks, nearest-even, one quantization for
#     both Fprop (as W^T) and Dgrad (as W);
#   * dY: 1x16 blocks, stochastic rounding (gradients); Dgrad draws with sr_seed, Wgrad's
#     dY^T with sr_seed + 1;
#   * the Hadamard transform goes on the Wgrad inputs only: X^T and dY^T along the token
#     dimension M, with one seed for both, so their product is unchanged.  The weight's
#     single quantization could not carry a transform along K for Fprop and along N for
#     Dgrad at once.
def linear_operands(x, w, dy, rht_seed: int, sr_seed: int):
    """Quantized operands of the three products, as ``quantize`` tuples:
    (X, W^T, W, dY, X^T, dY^T) for x (M, K), w (K, N), dy (M, N) bf16 bit patterns."""
    x, w, dy = (np.ascontiguousarray(a, dtype=np.uint16) for a in (x, w, dy))
    qx = quantize(x)
    qwt = quantize(np.ascontiguousarray(w.T), blocking=BLOCK_16x16)
    qw = quantize(w, blocking=BLOCK_16x16)
    qdy = quantize(dy, rounding=ROUND_SR, sr_seed=sr_seed)
    qxt = quantize(np.ascontiguousarray(x.T), rht=True, rht_seed=rht_seed)
    qdyt = quantize(np.ascontiguousarray(dy.T), rounding=ROUND_SR, rht=True, rht_seed=rht_seed,
                    sr_seed=sr_seed + 1)
    return qx, qwt, qw, qdy, qxt, qdyt


def linear_reference(x, w, dy, rht_seed: int, sr_seed: int, operands=None):
    """binary64 (Y, dX, dW) of the quantized linear layer (steps above)."""
    M, K = x.shape
    N = w.shape[1]
    qx, qwt, qw, qdy, qxt, qdyt = operands or linear_operands(x, w, dy, rht_seed, sr_seed)
    y = gemm_reference((*qx[:3], M, K, BLOCK_1x16), (*qwt[:3], N, K, BLOCK_16x16))
    dx = gemm_reference((*qdy[:3], M, N, BLOCK_1x16), (*qw[:3], K, N, BLOCK_16x16))
    dw = gemm_reference((*qxt[:3], K, M, BLOCK_1x16), (*qdyt[:3], N, M, BLOCK_1x16))
    return y, dx, dw
