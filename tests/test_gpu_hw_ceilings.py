"""Hardware ceilings the kernels are measured against (GPU, test-only microbenchmarks).

tests/native/hw_probe.hip times, on the box, the rates that the roofline figures of the
library are read against:

* the fp16 matrix-core instruction stream of the NVFP4 GEMM alone (its 256 x 256 tiles,
  128 x 128 per wave, v_mfma_f32_32x32x16_f16 on register-resident operands), over the
  FLOPs of the 8192 x 20480 x 5120 product, with random values shaped like dequantized
  NVFP4 elements, with zeros, and with the values of the workload-5 operands themselves:
  what the chip sustains under its power limit, against the 2.5 PFLOP/s dense fp16 figure;
* the same for the MXFP4 GEMM's scaled FP4 instruction, against the 10.1 PFLOP/s dense fp4
  figure;
* streaming HBM reads of the 84 MB activation tensor and streaming writes of 16-64 MiB with
  ordinary, non-temporal and write-through stores;
* the cost of one back-to-back launch of an empty kernel.

Each case prints its figure; the assertions only bound them loosely (a broken probe, not a
slow box, fails).  The probe is built by ``__graft_entry__.build()``.
"""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "tests", "native", "libhw_probe.so")
GEMM_FLOP = 2.0 * 8192 * 20480 * 5120
FP16_PEAK_TFLOPS = 2500.0
FP4_PEAK_TFLOPS = 10100.0
HBM_PEAK_GBPS = 8000.0


@pytest.fixture(scope="module")
def hwp():
    import torch
    assert torch.cuda.is_available()
    torch.cuda.init()
    if not os.path.exists(PROBE):
        pytest.fail("tests/native/libhw_probe.so is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(PROBE)
    i32, u64, d = ctypes.c_int, ctypes.c_uint64, ctypes.c_double
    L.hwp_mfma_stream.argtypes = [i32, i32, i32, i32, i32]
    L.hwp_read.argtypes = [u64, i32, i32, i32]
    L.hwp_write.argtypes = [u64, i32, i32, i32]
    L.hwp_empty.argtypes = [i32, i32]
    P = ctypes.c_void_p
    L.hwp_mfma_stream_operands.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32]
    L.hwp_mfma_fp4_stream.argtypes = [i32, i32, i32, P, P, P, P, i32, i32, i32, i32, i32]
    for f in (L.hwp_mfma_stream, L.hwp_read, L.hwp_write, L.hwp_empty, L.hwp_mfma_stream_operands,
              L.hwp_mfma_fp4_stream):
        f.restype = d
    return L


def test_mfma_stream_ceiling(hwp):
    """2560 tiles x 320 sub-steps of 16 MFMAs per wave = the workload-5 product's FLOPs.
    Each configuration: 20 untimed launches (the clocks settle), then three timings of 10
    launches; the best and the median are printed."""
    import numpy as np
    import torch
    from block_scaled_fp4_06_amd import nvfp4 as N
    from block_scaled_fp4_06_amd import workloads as W

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    # the workload-5 product's own operands (X with the transform, 1x16; W^T 16x16)
    qa = N.quantize(dev(W.w3()), rht=True, rht_seed=W.RHT_SEED)
    qw = N.quantize(dev(W.w5_weight()), blocking="16x16", with_transpose=True)
    b = qw.transposed()
    torch.cuda.synchronize()
    runs = {
        "mfma stream, random values": lambda warm: hwp.hwp_mfma_stream(2560, 320, 0, warm, 10),
        "mfma stream, zeros": lambda warm: hwp.hwp_mfma_stream(2560, 320, 1, warm, 10),
        "mfma stream, workload-5 operand values": lambda warm: hwp.hwp_mfma_stream_operands(
            qa.codes.data_ptr(), qa.scales.data_ptr(), b.codes.data_ptr(), b.scales.data_ptr(),
            8192, 20480, 5120, 320, warm, 10),
    }
    c = torch.empty(8192, 20480, dtype=torch.bfloat16, device="cuda")

    def gemm_us(warm):
        # the library's GEMM on the same operands, timed the same way
        for _ in range(warm):
            N.gemm(qa, b, torch.bfloat16, out=c)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            N.gemm(qa, b, torch.bfloat16, out=c)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 100.0
    runs["the NVFP4 GEMM itself (bf16 out)"] = gemm_us
    best = {}
    for name, run in runs.items():
        times = [run(20 if k == 0 else 2) for k in range(3)]
        assert min(times) > 0, "probe failed"
        best[name], med = min(times), float(np.median(times))
        tf = GEMM_FLOP / best[name] / 1e6
        print("%s: best %.1f us (median %.1f) per product, %.0f TFLOP/s, %.3f of the "
              "fp16 peak" % (name, best[name], med, tf, tf / FP16_PEAK_TFLOPS), flush=True)
        assert 0.2 * FP16_PEAK_TFLOPS < tf < 1.05 * FP16_PEAK_TFLOPS
    print("the GEMM runs at %.3f of the stream on its own operand values"
          % (best["mfma stream, workload-5 operand values"] / best["the NVFP4 GEMM itself (bf16 out)"]), flush=True)


def test_mfma_fp4_stream_ceiling(hwp):
    """The MXFP4 GEMM's instruction stream (v_mfma_scale_f32_32x32x64_f8f6f4, both operands
    FP4, register-resident) over the workload-5 product's FLOPs (2560 tiles x 80 sub-steps of
    K = 64), next to the library's MXFP4 GEMM on the workload-5 operands, against the 10.1
    PFLOP/s dense fp4 figure."""
    import numpy as np
    import torch
    from block_scaled_fp4_06_amd import nvfp4 as N
    from block_scaled_fp4_06_amd import workloads as W

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    qa = N.mx_quantize(dev(W.w3()))
    qb = N.mx_quantize(dev(np.ascontiguousarray(W.w5_weight().T)))
    torch.cuda.synchronize()
    ptrs = (qa.codes.data_ptr(), qa.scales.data_ptr(), qb.codes.data_ptr(), qb.scales.data_ptr())
    c = torch.empty(8192, 20480, dtype=torch.bfloat16, device="cuda")

    def gemm_us(warm):
        for _ in range(warm):
            N.mx_gemm(qa, qb, out=c)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            N.mx_gemm(qa, qb, out=c)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 100.0
    runs = {
        "fp4 mfma stream, random codes and scales":
            lambda warm: hwp.hwp_mfma_fp4_stream(2560, 80, 0, None, None, None, None, 0, 0, 0, warm, 10),
        "fp4 mfma stream, zeros":
            lambda warm: hwp.hwp_mfma_fp4_stream(2560, 80, 1, None, None, None, None, 0, 0, 0, warm, 10),
        "fp4 mfma stream, workload-5 MXFP4 operand values":
            lambda warm: hwp.hwp_mfma_fp4_stream(2560, 80, 2, *ptrs, 8192, 20480, 5120, warm, 10),
        "the MXFP4 GEMM itself (bf16 out)": gemm_us,
    }
    best = {}
    for name, run in runs.items():
        times = [run(20 if k == 0 else 2) for k in range(3)]
        assert min(times) > 0, "probe failed"
        best[name], med = min(times), float(np.median(times))
        tf = GEMM_FLOP / best[name] / 1e6
        print("%s: best %.1f us (median %.1f) per product, %.0f TFLOP/s, %.3f of the fp4 peak"
              % (name, best[name], med, tf, tf / FP4_PEAK_TFLOPS), flush=True)
        assert 0.05 * FP4_PEAK_TFLOPS < tf < 1.05 * FP4_PEAK_TFLOPS
    print("the MXFP4 GEMM runs at %.3f of the stream on its own operand values"
          % (best["fp4 mfma stream, workload-5 MXFP4 operand values"]
             / best["the MXFP4 GEMM itself (bf16 out)"]), flush=True)


def test_hbm_read_write_rates(hwp):
    nbytes = 8192 * 5120 * 2   # the 84 MB activation tensor
    for wgs in (1024, 10240):
        us = hwp.hwp_read(nbytes, 7, wgs, 70)
        assert us > 0, "probe failed"
        gbps = nbytes / us / 1e3
        print("read %d MB, %5d workgroups: %.2f us per launch, %.0f GB/s (%.3f of 8 TB/s)"
              % (nbytes // 1000000, wgs, us, gbps, gbps / HBM_PEAK_GBPS), flush=True)
        assert 1000 < gbps < 1.05 * HBM_PEAK_GBPS
    names = ("ordinary", "non-temporal", "write-through (sc1)")
    for mib in (16, 24, 64):
        for pol in (0, 1, 2):
            us = hwp.hwp_write(mib << 20, pol, 1024, 50)
            assert us > 0, "probe failed"
            gbps = (mib << 20) / us / 1e3
            print("write %2d MiB, %-19s stores: %.2f us per launch, %.0f GB/s"
                  % (mib, names[pol], us, gbps), flush=True)
            assert gbps < 1.05 * HBM_PEAK_GBPS


def test_launch_cost(hwp):
    for wgs in (256, 1024):
        us = hwp.hwp_empty(wgs, 100)
        assert us > 0, "probe failed"
        print("empty kernel, %4d workgroups: %.2f us per back-to-back launch" % (wgs, us), flush=True)
        assert us < 50
