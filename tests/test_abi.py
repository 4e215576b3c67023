"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function include/nvfp4.h declares, and reject bad
arguments with the documented status before it makes any HIP call -- so these calls
use fake (but aligned) addresses and never reach a kernel launch.
"""
import ctypes
import os
import re

import pytest

from block_scaled_fp4_06_amd import nvfp4 as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

FAKE = 0x10000  # aligned, never dereferenced: validation fails before any use
ERR = dict(OK=0, NULL=1, SHAPE=2, ALIGN=3, UNSUPPORTED=4, WORKSPACE=5, HIP=6)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(N.LIB_PATH):
        from block_scaled_fp4_06_amd import build
        build.build()
    return N.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b((?:nv|mx)fp4_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(N.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_strings(lib):
    assert N.nvfp4_abi_version() == 1
    for s in range(7):
        assert N.nvfp4_status_string(s)
    assert "unknown" in N.nvfp4_status_string(99)
    assert N.nvfp4_quantize_workspace_bytes() >= 4096


def q(params=None, x=FAKE, rows=32, cols=32, ld=32, codes=FAKE, scales=FAKE, g=FAKE,
      ct=None, st=None, status=None, ws=FAKE, wsb=None):
    if params is None:
        params = N.QuantParams(0, 0, 0, 0, 0, 0, 0)
    if wsb is None:
        wsb = N.nvfp4_quantize_workspace_bytes()
    return N.nvfp4_quantize(x, rows, cols, ld, params, codes, scales, g, ct, st, status, ws,
                            wsb, None)


def test_quantize_argument_errors(lib):
    P = N.QuantParams
    assert q(x=None) == ERR["NULL"]
    assert q(codes=None) == ERR["NULL"]
    assert q(scales=None) == ERR["NULL"]
    assert q(g=None) == ERR["NULL"]
    assert q(rows=24) == ERR["SHAPE"]
    assert q(cols=40, ld=40) == ERR["SHAPE"]
    assert q(rows=-16) == ERR["SHAPE"]
    assert q(ld=16) == ERR["SHAPE"]
    assert q(ld=36) == ERR["ALIGN"]
    assert q(x=FAKE + 8) == ERR["ALIGN"]
    assert q(codes=FAKE + 4) == ERR["ALIGN"]
    assert q(ws=None) == ERR["WORKSPACE"]
    assert q(wsb=16) == ERR["WORKSPACE"]
    assert q(P(2, 0, 0, 0, 0, 0, 0)) == ERR["UNSUPPORTED"]
    assert q(P(0, 3, 0, 0, 0, 0, 0)) == ERR["UNSUPPORTED"]
    assert q(P(0, 0, 2, 0, 0, 0, 0)) == ERR["UNSUPPORTED"]
    assert q(P(0, 0, 0, 1, 0, 0, 0)) == ERR["UNSUPPORTED"]
    assert q(P(0, 1, 0, 0, 0, 0, 8)) == ERR["SHAPE"]        # SR base not a multiple of 16
    assert q(ct=FAKE) == ERR["NULL"]                         # codes_t without scales_t
    assert q(ct=FAKE, st=FAKE) == ERR["UNSUPPORTED"]         # transpose needs 16x16
    assert q(status=FAKE + 2) == ERR["ALIGN"]


def test_quantize_null_params(lib):
    L = lib
    rc = L.nvfp4_quantize(FAKE, 16, 16, 16, None, FAKE, FAKE, FAKE, None, None, None, FAKE,
                          1 << 20, None)
    assert rc == ERR["NULL"]


def test_dequantize_argument_errors(lib):
    def d(codes=FAKE, scales=FAKE, g=FAKE, rows=32, cols=32, blk=0, y=FAKE, ld=32, od=0):
        return N.nvfp4_dequantize(codes, scales, g, rows, cols, blk, y, ld, od, None)
    assert d(codes=None) == ERR["NULL"]
    assert d(y=None) == ERR["NULL"]
    assert d(g=None) == ERR["NULL"]
    assert d(rows=8) == ERR["SHAPE"]
    assert d(ld=16) == ERR["SHAPE"]
    assert d(ld=44) == ERR["ALIGN"]
    assert d(y=FAKE + 2) == ERR["ALIGN"]
    assert d(blk=5) == ERR["UNSUPPORTED"]
    assert d(od=2) == ERR["UNSUPPORTED"]
    # an empty tensor is a no-op that needs no pointers (and makes no HIP call)
    assert d(rows=0, codes=None, scales=None, g=None, y=None) == ERR["OK"]


def test_gemm_argument_errors(lib):
    def op(codes=FAKE, scales=FAKE, g=FAKE, blk=0, res=0):
        return N.Operand(codes, scales, g, blk, res)

    def gm(a=None, b=None, M=32, N_=32, K=64, c=FAKE, ldc=32, od=0):
        a = a or op()
        b = b or op(blk=1)
        return N.nvfp4_gemm(a, b, M, N_, K, c, ldc, od, None)
    assert lib.nvfp4_gemm(None, None, 16, 16, 16, FAKE, 16, 0, None) == ERR["NULL"]
    assert gm(a=op(codes=None)) == ERR["NULL"]
    assert gm(b=op(g=None)) == ERR["NULL"]
    assert gm(c=None) == ERR["NULL"]
    assert gm(K=40) == ERR["SHAPE"]
    assert gm(K=1 << 24) == ERR["SHAPE"]
    assert gm(M=1 << 30, N_=1 << 30, ldc=1 << 30) == ERR["SHAPE"]   # 2^40 tiles of C
    assert gm(M=-16) == ERR["SHAPE"]
    assert gm(ldc=16) == ERR["SHAPE"]
    assert gm(ldc=36) == ERR["ALIGN"]
    assert gm(a=op(scales=FAKE + 1)) == ERR["ALIGN"]
    assert gm(a=op(blk=7)) == ERR["UNSUPPORTED"]
    assert gm(b=op(res=1)) == ERR["UNSUPPORTED"]
    assert gm(od=9) == ERR["UNSUPPORTED"]
    assert gm(M=0, a=op(codes=None, scales=None, g=None), c=None) == ERR["OK"]


def test_gemm_ws_argument_errors(lib):
    wsb = N.nvfp4_gemm_workspace_bytes()
    # counters plus 256 partial tiles of 256 x 256 fp32
    assert wsb == 4096 + 256 * 256 * 256 * 4

    def op(codes=FAKE, scales=FAKE, g=FAKE, blk=0):
        return N.Operand(codes, scales, g, blk, 0)

    def gm(ws=FAKE, nbytes=wsb, M=32, K=64, c=FAKE, ldc=32, a=None):
        return N.nvfp4_gemm_ws(a or op(), op(blk=1), M, 32, K, c, ldc, 0, ws, nbytes, None)
    assert gm(ws=None) == ERR["WORKSPACE"]
    assert gm(nbytes=wsb - 1) == ERR["WORKSPACE"]
    assert gm(ws=FAKE + 8) == ERR["ALIGN"]
    # then the checks of nvfp4_gemm
    assert gm(K=40) == ERR["SHAPE"]
    assert gm(c=None) == ERR["NULL"]
    assert gm(ldc=36) == ERR["ALIGN"]
    assert gm(a=op(codes=None)) == ERR["NULL"]
    assert gm(M=0, c=None) == ERR["OK"]


def test_mx_argument_errors(lib):
    def q(x=FAKE, rows=32, cols=64, ld=64, codes=FAKE, scales=FAKE):
        return N.mxfp4_quantize(x, rows, cols, ld, codes, scales, None)
    assert q(x=None) == ERR["NULL"]
    assert q(scales=None) == ERR["NULL"]
    assert q(cols=48, ld=48) == ERR["SHAPE"]          # blocks are 32 elements
    assert q(rows=-1) == ERR["SHAPE"]
    assert q(ld=32) == ERR["SHAPE"]
    assert q(ld=68) == ERR["ALIGN"]
    assert q(codes=FAKE + 4) == ERR["ALIGN"]
    assert q(rows=1 << 20, cols=1 << 15, ld=1 << 15) == ERR["SHAPE"]   # 2^35 elements
    assert q(rows=0, x=None, codes=None, scales=None) == ERR["OK"]

    def d(codes=FAKE, scales=FAKE, rows=32, cols=64, y=FAKE, ld=64, od=0):
        return N.mxfp4_dequantize(codes, scales, rows, cols, y, ld, od, None)
    assert d(codes=None) == ERR["NULL"]
    assert d(y=None) == ERR["NULL"]
    assert d(cols=16, ld=16) == ERR["SHAPE"]
    assert d(ld=60) == ERR["SHAPE"]
    assert d(ld=68) == ERR["ALIGN"]
    assert d(od=3) == ERR["UNSUPPORTED"]
    assert d(cols=0, codes=None, scales=None, y=None) == ERR["OK"]

    def gm(ac=FAKE, as_=FAKE, bc=FAKE, bs=FAKE, M=32, N_=32, K=64, c=FAKE, ldc=32, od=0):
        return N.mxfp4_gemm(ac, as_, bc, bs, M, N_, K, c, ldc, od, None)
    assert gm(ac=None) == ERR["NULL"]
    assert gm(bs=None) == ERR["NULL"]
    assert gm(c=None) == ERR["NULL"]
    assert gm(K=48) == ERR["SHAPE"]
    assert gm(K=1 << 24) == ERR["SHAPE"]
    assert gm(M=1 << 24, N_=1 << 24, ldc=1 << 24) == ERR["SHAPE"]   # 2^34 tiles of C
    assert gm(M=-1) == ERR["SHAPE"]
    assert gm(ldc=16) == ERR["SHAPE"]
    assert gm(as_=FAKE + 1) == ERR["ALIGN"]
    assert gm(od=2) == ERR["UNSUPPORTED"]
    assert gm(N_=0, ac=None, as_=None, bc=None, bs=None, c=None) == ERR["OK"]


def test_transpose_argument_errors(lib):
    def t(x=FAKE, rows=32, cols=64, ldx=64, y=FAKE, ldy=32):
        return N.nvfp4_transpose_bf16(x, rows, cols, ldx, y, ldy, None)
    assert t(x=None) == ERR["NULL"]
    assert t(y=None) == ERR["NULL"]
    assert t(rows=12) == ERR["SHAPE"]
    assert t(cols=60, ldx=60) == ERR["SHAPE"]
    assert t(ldx=32) == ERR["SHAPE"]
    assert t(ldy=16) == ERR["SHAPE"]
    assert t(ldx=68) == ERR["ALIGN"]
    assert t(y=FAKE + 8) == ERR["ALIGN"]
    assert t(rows=0, x=None, y=None) == ERR["OK"]


# Shapes whose element count overflows a 64-bit product (2^68), wraps to zero (2^64) or
# wraps to exactly 2^35 ((2^33 + 16) * 2^31 = 2^64 + 2^35), and one just above 2^35.
HUGE = [(1 << 34, 1 << 34), (1 << 32, 1 << 32), ((1 << 33) + 16, 1 << 31), ((1 << 35) + 16, 1 << 4),
        (1 << 20, (1 << 15) + 16)]


@pytest.mark.parametrize("rows,cols", HUGE)
def test_huge_shapes_rejected_without_overflow(lib, rows, cols):
    P = N.QuantParams
    for prm in (P(0, 0, 0, 0, 0, 0, 0), P(0, 1, 0, 0, 0, 0, 0), P(0, 0, 1, 0, 0, 0, 0),
                P(1, 0, 0, 0, 0, 0, 0), P(1, 1, 1, 0, 0, 0, 0)):
        assert q(prm, rows=rows, cols=cols, ld=cols) == ERR["SHAPE"], (rows, cols, prm.blocking)
    assert q(P(1, 0, 0, 0, 0, 0, 0), rows=rows, cols=cols, ld=cols, ct=FAKE,
             st=FAKE) == ERR["SHAPE"]
    for blk in (0, 1):
        for od in (0, 1):
            assert N.nvfp4_dequantize(FAKE, FAKE, FAKE, rows, cols, blk, FAKE, cols, od,
                                      None) == ERR["SHAPE"]
    mcols = cols - (cols & 31)   # MXFP4 blocks are 32 elements
    if mcols:
        assert N.mxfp4_quantize(FAKE, rows, mcols, mcols, FAKE, FAKE, None) == ERR["SHAPE"]
        assert N.mxfp4_dequantize(FAKE, FAKE, rows, mcols, FAKE, mcols, 0, None) == ERR["SHAPE"]
    assert N.nvfp4_transpose_bf16(FAKE, rows, cols, cols, FAKE, rows, None) == ERR["SHAPE"]


def test_leading_dimension_overflow_rejected(lib):
    # a small tensor whose row stride makes (rows - 1) * ld overflow 64-bit offsets
    big = 1 << 62
    assert q(rows=32, cols=32, ld=big) == ERR["SHAPE"]
    assert N.nvfp4_dequantize(FAKE, FAKE, FAKE, 32, 32, 0, FAKE, big, 0, None) == ERR["SHAPE"]
    assert N.mxfp4_quantize(FAKE, 32, 64, big, FAKE, FAKE, None) == ERR["SHAPE"]
    assert N.mxfp4_dequantize(FAKE, FAKE, 32, 64, FAKE, big, 0, None) == ERR["SHAPE"]
    assert N.nvfp4_transpose_bf16(FAKE, 32, 64, big, FAKE, 32, None) == ERR["SHAPE"]
    assert N.nvfp4_transpose_bf16(FAKE, 32, 64, 64, FAKE, big, None) == ERR["SHAPE"]
    op = N.Operand(FAKE, FAKE, FAKE, 0, 0)
    assert N.nvfp4_gemm(op, op, 32, 32, 64, FAKE, big, 0, None) == ERR["SHAPE"]
    assert N.mxfp4_gemm(FAKE, FAKE, FAKE, FAKE, 32, 32, 64, FAKE, big, 0, None) == ERR["SHAPE"]
    # a stride just below the largest whose span (rows - 1) * ld + cols stays within 2^60
    # elements passes the shape checks (and then fails on alignment); the next multiple of 8
    # above the largest does not
    ld_max = ((1 << 60) - 16) // 15
    assert ld_max % 8 == 0
    assert q(rows=16, cols=16, ld=ld_max - 1) == ERR["ALIGN"]
    assert q(rows=16, cols=16, ld=ld_max + 8) == ERR["SHAPE"]


def test_python_wrapper_raises_when_library_missing(tmp_path, monkeypatch):
    monkeypatch.setattr(N, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        N.load(str(tmp_path / "missing.so"))
