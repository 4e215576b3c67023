"""Phase timeline of the quantize kernels on the workloads.

A test-only variant of the library (tests/native/libnvfp4_timeline.so, built by
__graft_entry__.build() from the same sources with NVFP4_TIMELINE) records, per workgroup,
the constant 100 MHz clock at the phase boundaries of each quantize kernel: start, own
partial maxima published, tensor amax known, end.  These tests run one launch of each
workload under it, check that the stamps are ordered and that the instrumented library
quantizes exactly like the product library, and print the phase table (run with -s).
"""
import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
TL_LIB = os.path.join(HERE, "native", "libnvfp4_timeline.so")
WGS = 8192                       # workgroups per region (kTlWgs)
REGIONS = {"fused_1x16": 0, "16x16": 1, "amax_pass": 2, "sr_pass2": 3}
TICK_US = 0.01                   # 100 MHz


@pytest.fixture(scope="module")
def tl():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(TL_LIB):
        pytest.fail("timeline library not built: run __graft_entry__.build()")
    from block_scaled_fp4_06_amd import nvfp4 as N
    N.load()
    L = ctypes.CDLL(TL_LIB)
    P, i64 = ctypes.c_void_p, ctypes.c_int64
    L.nvfp4_quantize.argtypes = [P, i64, i64, i64, ctypes.POINTER(N.QuantParams), P, P, P, P,
                                 P, P, P, ctypes.c_size_t, P]
    L.nvfp4_quantize.restype = ctypes.c_int
    L.nvfp4_timeline_attach.argtypes = [P]
    L.nvfp4_timeline_attach.restype = ctypes.c_int
    return L


def _run(L, x, blocking, rounding, rht, with_t):
    """One instrumented launch after three warm ones: (stamps[4, WGS, 4], event ms, outputs)."""
    import torch
    from block_scaled_fp4_06_amd import nvfp4 as N
    from block_scaled_fp4_06_amd import workloads as W
    rows, cols = x.shape
    dev = x.device
    blk = 1 if blocking == "16x16" else 0
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows // 16, cols // 16) if blk else (rows, cols // 16),
                         dtype=torch.uint8, device=dev)
    g = torch.empty(1, dtype=torch.float32, device=dev)
    ct = st = None
    if with_t:
        ct = torch.empty((cols, rows // 2), dtype=torch.uint8, device=dev)
        st = torch.empty((cols // 16, rows // 16), dtype=torch.uint8, device=dev)
    ws = N.new_workspace(dev)
    buf = torch.zeros(len(REGIONS) * WGS * 4, dtype=torch.int64, device=dev)
    prm = N.QuantParams(blk, 1 if rounding == "sr" else 0, 1 if rht else 0, 0,
                        W.RHT_SEED if rht else 0, 7, 0)
    s = torch.cuda.current_stream().cuda_stream

    def call():
        rc = L.nvfp4_quantize(x.data_ptr(), rows, cols, x.stride(0), ctypes.byref(prm),
                              codes.data_ptr(), scales.data_ptr(), g.data_ptr(),
                              ct.data_ptr() if with_t else None,
                              st.data_ptr() if with_t else None, None, ws.data_ptr(),
                              ws.numel(), s)
        assert rc == 0, rc

    assert L.nvfp4_timeline_attach(buf.data_ptr()) == 0
    try:
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        buf.zero_()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
    finally:
        assert L.nvfp4_timeline_attach(None) == 0
    stamps = buf.cpu().numpy().reshape(len(REGIONS), WGS, 4)
    return stamps, e0.elapsed_time(e1), (codes, scales, g, ct, st)


def _phases(stamps, region, t0):
    """Per-phase (min, median, max) in us from t0 over the workgroups of a region."""
    st = stamps[region]
    used = st[:, 0] != 0
    st = st[used]
    out = {"wgs": int(used.sum())}
    for i, name in enumerate(("start", "published", "amax_known", "end")):
        col = st[:, i]
        if (col != 0).all():
            us = (col - t0) * TICK_US
            out[name] = (float(us.min()), float(np.median(us)), float(us.max()))
    return out


def _check_order(stamps, region, idx):
    st = stamps[region]
    st = st[st[:, 0] != 0]
    assert len(st) > 0
    for a, b in zip(idx, idx[1:]):
        assert (st[:, a] <= st[:, b]).all(), (region, a, b)


def _fmt(name, ph):
    parts = ["%-40s wgs %5d" % (name, ph["wgs"])]
    for k in ("start", "published", "amax_known", "end"):
        if k in ph:
            parts.append("%s %.2f/%.2f/%.2f" % (k, *ph[k]))
    return "  ".join(parts)


CASES = [
    ("W3 8192x5120 1x16 RHT RNE", "w3", "1x16", "rne", True, False),
    ("W2 4096x4096 16x16 + W^T", "w2", "16x16", "rne", False, True),
    ("W5 weight 5120x20480 16x16 + W^T", "w5_weight", "16x16", "rne", False, True),
    ("W4 8192x5120 1x16 RHT SR", "w4", "1x16", "sr", True, False),
]


@pytest.mark.parametrize("name,gen,blocking,rounding,rht,with_t", CASES,
                         ids=[c[1] for c in CASES])
def test_phase_timeline(tl, name, gen, blocking, rounding, rht, with_t):
    import torch
    from block_scaled_fp4_06_amd import nvfp4 as N
    from block_scaled_fp4_06_amd import workloads as W
    xh = getattr(W, gen)()
    x = torch.from_numpy(np.ascontiguousarray(xh).view(np.int16)).view(torch.bfloat16).cuda()
    stamps, ms, (codes, scales, g, ct, st) = _run(tl, x, blocking, rounding, rht, with_t)
    # the instrumented library quantizes exactly like the product one
    q = N.quantize(x, blocking=blocking, rounding=rounding, rht=rht,
                   rht_seed=W.RHT_SEED if rht else 0, sr_seed=7, with_transpose=with_t)
    torch.cuda.synchronize()
    assert torch.equal(q.codes, codes) and torch.equal(q.scales, scales)
    assert torch.equal(q.global_dec, g)
    if with_t:
        assert torch.equal(q.codes_t, ct) and torch.equal(q.scales_t, st)
    lines = ["%s: one launch %.2f us (events)" % (name, ms * 1000)]
    if rounding == "sr":
        r1, r2 = REGIONS["amax_pass"], REGIONS["sr_pass2"]
        _check_order(stamps, r1, (0, 1, 3))
        _check_order(stamps, r2, (0, 2, 3))
        used = np.concatenate([stamps[r][stamps[r][:, 0] != 0, 0] for r in (r1, r2)])
        t0 = int(used.min())
        lines.append(_fmt("  pass 1 (amax_kernel)", _phases(stamps, r1, t0)))
        lines.append(_fmt("  pass 2 (quant_1x16_sr_kernel)", _phases(stamps, r2, t0)))
    else:
        r = REGIONS["fused_1x16" if blocking == "1x16" else "16x16"]
        _check_order(stamps, r, (0, 1, 2, 3))
        t0 = int(stamps[r][stamps[r][:, 0] != 0, 0].min())
        lines.append(_fmt("  fused kernel", _phases(stamps, r, t0)))
    print("\n" + "\n".join(lines), flush=True)
