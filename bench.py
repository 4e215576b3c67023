"""Benchmark of the NVFP4 hot path on one MI355X.

One step = one NVFP4 linear-layer pass over the workload-5 shapes, every kernel of the
path once:
  quantize X   8192 x 5120 bf16 activations, 16-point RHT + 1x16 blocks, nearest-even
  quantize W   5120 x 20480 bf16 weight, 16x16 blocks, W and W^T codes from one read
  GEMM         C = X_q . (W^T)_q^T, 8192 x 20480 x 5120, fp32 accumulate, bf16 out
  dequantize   X_q -> bf16
Inputs are seeded synthetic tensors resident in HBM before timing starts.  The timed
steps are replays of a HIP graph of one step, so the step time is GPU time.  The printed
JSON line carries the step throughput (GEMM FLOP per step / step time), per-kernel times
(HIP events around a graph of back-to-back launches of that kernel, on the stream it runs
on), the roofline of the dominant kernel, standalone quantize figures for workloads 2-4 (input buffers rotated so the
256 MB Infinity Cache cannot hold them), the MXFP4 variant (quantize, and the GEMM on the
native scaled FP4 MFMA), one linear-layer training step (Fprop, Dgrad, Wgrad), and the
CPU oracle's rate on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-micro]
    python bench.py --summarize ROCPROF_DIR [--last N]   (summary of a rocprofv3 csv run)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix peak
MFMA_FP4_PEAK_TFLOPS = 10100.0  # dense fp4 (context only: NVFP4's E4M3-per-16 scales
                                # cannot be applied by gfx950's E8M0-per-32 FP4 MFMA)
METRIC = "NVFP4 quantize GB/s (% HBM peak); NVFP4 GEMM TFLOP/s (% MFMA peak)"
M, K, NN = 8192, 5120, 20480


def quant_bytes(rows, cols, blocking, transpose=False):
    """Algorithmic bytes: bf16 input read once + packed codes + E4M3 scales + 4 B."""
    n = rows * cols
    sc = n // 256 if blocking == "16x16" else n // 16
    out = n // 2 + sc
    return 2 * n + out * (2 if transpose else 1) + 4


def dequant_bytes(rows, cols, blocking, out_bytes=2):
    n = rows * cols
    sc = n // 256 if blocking == "16x16" else n // 16
    return n // 2 + sc + 4 + n * out_bytes


def gemm_traffic_bytes():
    """HBM bytes of one GEMM launch measured with rocprofv3 (FETCH_SIZE x2, WRITE_SIZE x1,
    scales from a plain-copy calibration), or None when the kernel source has changed since
    the counters were taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    rec_path = os.path.join(here, "profiles", "gemm_w5_traffic.json")
    src_path = os.path.join(here, "block_scaled_fp4_06_amd", "csrc", "gemm.hip")
    try:
        rec = json.load(open(rec_path))
        src = hashlib.sha256(open(src_path, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    return int(rec["traffic_bytes"]) if rec.get("source_sha256") == src else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the clocks settle over the first ~15 GEMMs (1.6-1.7 ms falling to ~1.3 ms), so the
    # default warm-up runs 20 steps (~30 ms) before timing
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-micro", action="store_true")
    ap.add_argument("--context", action="store_true", help="also time torch fp16 matmul")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM counters)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="print the summary of a rocprofv3 output directory (kernel trace "
                         "and/or counters) instead of benchmarking")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/gemm_w5_traffic.json from two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, WRITE_SIZE) of a bench run with --copy-calibration")
    ap.add_argument("--last", type=int, default=0,
                    help="with --summarize: only the last N dispatches of each kernel and "
                         "grid (the timed ones of a run with --steps N)")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def to_dev(x_u16):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_u16).view(np.int16)).view(torch.bfloat16).cuda()


def copy_bandwidth(nbuf_bytes=512 << 20, chunk=84 << 20, iters=30):
    """Device-to-device copy rate (GB/s, read + write bytes) over rotated buffers: the
    practical HBM ceiling the quantize rates are also compared with."""
    import torch
    nb = max(2, -(-nbuf_bytes // chunk))
    src = [torch.empty(chunk, dtype=torch.uint8, device="cuda") for _ in range(nb)]
    dst = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    for i in range(5):
        dst.copy_(src[i % nb])
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(iters):
        dst.copy_(src[i % nb])
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1000.0 / iters
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * chunk / us / 1e3, 1)


def micro_quantize(N, W, nbuf_bytes=512 << 20, iters=30, reps=7, copy_gbps=None):
    """Standalone quantize of workloads 2-4 (and workload 2 with the RHT) with rotated
    input buffers; median and p10/p90 over `reps` replays of `iters` graph-captured calls."""
    import torch
    res = {}
    cases = [
        ("w2_16x16_wt", W.w2(), dict(blocking="16x16", with_transpose=True), "16x16", True),
        ("w3_rht_1x16_rne", W.w3(), dict(rht=True, rht_seed=W.RHT_SEED), "1x16", False),
        ("w4_rht_1x16_sr", W.w4(), dict(rht=True, rht_seed=W.RHT_SEED, rounding="sr", sr_seed=7),
         "1x16", False),
        # weight with the activations' transform along K (both GEMM operands transformed)
        ("w2_rht_16x16_wt", W.w2(), dict(blocking="16x16", with_transpose=True, rht=True,
                                         rht_seed=W.RHT_SEED), "16x16", True),
    ]
    for name, x, kw, blk, tr in cases:
        xd = to_dev(x)
        nb = max(2, -(-nbuf_bytes // (xd.numel() * 2)))
        bufs = [xd] + [xd.clone() for _ in range(nb - 1)]
        ws = N.new_workspace(xd.device)
        q = N.quantize(xd, workspace=ws, **kw)
        for i in range(5):
            N.quantize(bufs[i % nb], out=q, workspace=ws, **kw)
        torch.cuda.synchronize()
        # the timed launches are replayed from a captured graph, so that the host's
        # per-call cost (Python and ctypes) never leaves the GPU idle between kernels
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=torch.cuda.Stream()):
            for i in range(iters):
                N.quantize(bufs[i % nb], out=q, workspace=ws, **kw)
        g.replay()
        torch.cuda.synchronize()
        per = []
        for _ in range(reps):   # each replay: the mean over `iters` calls
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            per.append(a.elapsed_time(b) * 1000.0 / iters)
        p10, us, p90 = (float(v) for v in np.percentile(per, [10, 50, 90]))
        by = quant_bytes(x.shape[0], x.shape[1], blk, tr)
        res[name] = {"us": round(us, 2), "us_p10": round(p10, 2), "us_p90": round(p90, 2),
                     "GBps": round(by / us / 1e3, 1),
                     "frac": round(by / us / 1e3 / HBM_PEAK_GBPS, 4), "bytes": by,
                     "buffers": nb}
        if copy_gbps:
            res[name]["frac_copy"] = round(by / us / 1e3 / copy_gbps, 4)
        log("micro %s: %.2f us (p10 %.2f, p90 %.2f), %.1f GB/s" % (name, us, p10, p90, by / us / 1e3))
        del bufs, xd, q, g, ws
        torch.cuda.empty_cache()
    return res


def micro_mxfp4(N, W, nbuf_bytes=512 << 20, iters=30, gemm_iters=10, copy_gbps=None):
    """MXFP4 (32-element E8M0 blocks): quantize of workload 3 (rotated input buffers,
    graph-replayed) and the workload-5 GEMM on the native scaled FP4 MFMA."""
    import torch
    res = {}
    xd = to_dev(W.w3())
    n = xd.numel()
    nb = max(2, -(-nbuf_bytes // (n * 2)))
    bufs = [xd] + [xd.clone() for _ in range(nb - 1)]
    q = N.mx_quantize(xd)
    for i in range(5):
        N.mx_quantize(bufs[i % nb], out=q)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        for i in range(iters):
            N.mx_quantize(bufs[i % nb], out=q)
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1000.0 / iters
    by = 2 * n + n // 2 + n // 32
    res["mx_quantize_w3"] = {"us": round(us, 2), "GBps": round(by / us / 1e3, 1),
                             "frac": round(by / us / 1e3 / HBM_PEAK_GBPS, 4), "bytes": by,
                             "buffers": nb}
    if copy_gbps:
        res["mx_quantize_w3"]["frac_copy"] = round(by / us / 1e3 / copy_gbps, 4)
    log("micro mx_quantize_w3: %.2f us, %.1f GB/s" % (us, by / us / 1e3))
    del bufs, g
    wt = to_dev(np.ascontiguousarray(W.w5_weight().T))
    qa, qb = N.mx_quantize(xd), N.mx_quantize(wt)
    C = torch.empty((M, NN), dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        N.mx_gemm(qa, qb, out=C)
    torch.cuda.synchronize()
    a.record()
    for _ in range(gemm_iters):
        N.mx_gemm(qa, qb, out=C)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1000.0 / gemm_iters
    tf = 2.0 * M * NN * K / us / 1e6
    res["mx_gemm_w5"] = {"us": round(us, 1), "TFLOPs": round(tf, 1),
                         "frac_mfma_fp4": round(tf / MFMA_FP4_PEAK_TFLOPS, 4)}
    log("micro mx_gemm_w5: %.1f us, %.1f TFLOP/s" % (us, tf))
    del xd, wt, qa, qb, C
    torch.cuda.empty_cache()
    return res


def micro_linear(N, W, steps=5, warmup=2):
    """One NVFP4 linear-layer training step at the workload-5 sizes: Fprop, Dgrad, Wgrad
    with their quantizations and the two transposes of the Wgrad inputs."""
    import torch
    from block_scaled_fp4_06_amd import linear as L
    x = to_dev(W.w3())
    w = to_dev(W.w5_weight())
    dy = to_dev(W.student_t(M, NN, seed=6))
    for _ in range(warmup):
        y, ctx = L.linear_forward(x, w)
        L.linear_backward(dy, ctx)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    fwd = bwd = 0.0
    for _ in range(steps):
        ev[0].record()
        y, ctx = L.linear_forward(x, w)
        ev[1].record()
        dx, dw = L.linear_backward(dy, ctx)
        ev[2].record()
        torch.cuda.synchronize()
        fwd += ev[0].elapsed_time(ev[1])
        bwd += ev[1].elapsed_time(ev[2])
    fwd, bwd = fwd / steps, bwd / steps
    flops = 3 * 2.0 * M * NN * K
    res = {"ms_fwd": round(fwd, 3), "ms_bwd": round(bwd, 3),
           "TFLOPs_step": round(flops / ((fwd + bwd) * 1e-3) / 1e12, 1)}
    log("micro linear layer step: fwd %.3f ms, bwd %.3f ms" % (fwd, bwd))
    del x, w, dy, y, ctx, dx, dw
    torch.cuda.empty_cache()
    return res


def context_scaled_mm_mx(N, W, iters=10):
    """torch's scaled_mm (hipBLASLt) on MXFP4 operands from this library's quantizer, for
    comparison with mxfp4_gemm on the same data; None where unsupported."""
    import torch
    import torch.nn.functional as F
    try:
        qa = N.mx_quantize(to_dev(W.w3()))
        qb = N.mx_quantize(to_dev(np.ascontiguousarray(W.w5_weight().T)))
        ST = getattr(F, "ScalingType", None) or F._ScalingType
        SW = getattr(F, "SwizzleType", None) or F._SwizzleType
        args = (qa.codes.view(torch.float4_e2m1fn_x2), qb.codes.view(torch.float4_e2m1fn_x2).t(),
                qa.scales.view(torch.float8_e8m0fnu), ST.BlockWise1x32,
                qb.scales.view(torch.float8_e8m0fnu), ST.BlockWise1x32, SW.NO_SWIZZLE,
                SW.NO_SWIZZLE)

        def call():
            return F.scaled_mm(args[0], args[1], args[2], args[3], args[4], args[5], args[6],
                               args[7], output_dtype=torch.bfloat16)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(iters):
            call()
        b.record()
        torch.cuda.synchronize()
        return round(2.0 * M * NN * K / (a.elapsed_time(b) / iters * 1e-3) / 1e12, 1)
    except (RuntimeError, AttributeError, TypeError) as e:
        log("scaled_mm MXFP4 unavailable: %s" % str(e)[:200])
        return None


def cpu_baseline(x_np, w_np, sample_rows=M, repeats=5):
    """The oracle timed on this host: one step (quantize X and W with W^T, the binary64
    GEMM, dequantize X) on `sample_rows` of the 8192 activation rows (all by default),
    the rows' share scaled to a step; the median of `repeats` runs."""
    import oracle
    from block_scaled_fp4_06_amd import workloads as W
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    cores = min(threads, os.cpu_count() or 1)
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    xs = np.ascontiguousarray(x_np[:sample_rows])
    steps, work = [], 0.0
    for _ in range(repeats):
        t0 = time.perf_counter()
        ca, sa, ga, _ = oracle.quantize(xs, rht=True, rht_seed=W.RHT_SEED)
        t1 = time.perf_counter()
        cw, sw, gw, _ = oracle.quantize(w_np, blocking=oracle.BLOCK_16x16)
        wt = np.ascontiguousarray(w_np.T)
        cwt, swt, _, _ = oracle.quantize(wt, blocking=oracle.BLOCK_16x16)
        t2 = time.perf_counter()
        c = oracle.gemm_reference((ca, sa, ga, sample_rows, K, 0), (cwt, swt, gw, NN, K, 1))
        t3 = time.perf_counter()
        oracle.dequantize_bf16(ca, sa, ga, sample_rows, K)
        t4 = time.perf_counter()
        del c, wt
        scale = M / sample_rows
        steps.append((t1 - t0) * scale + (t2 - t1) + (t3 - t2) * scale + (t4 - t3) * scale)
        work += t4 - t0
    t_step = float(np.median(steps))
    flops = 2.0 * M * NN * K
    # the activation quantize alone, on one thread and on all of them (GB/s by the
    # algorithmic bytes of the sample)
    rates = {}
    try:
        import ctypes
        gomp = ctypes.CDLL("libgomp.so.1")
        xq = np.ascontiguousarray(x_np[:1024])
        by = quant_bytes(1024, K, "1x16")
        for n in (1, threads):
            gomp.omp_set_num_threads(n)
            t0 = time.perf_counter()
            oracle.quantize(xq, rht=True, rht_seed=W.RHT_SEED)
            rates["quantize_x_GBps_%d_thread%s" % (n, "" if n == 1 else "s")] = round(
                by / (time.perf_counter() - t0) / 1e9, 3)
        gomp.omp_set_num_threads(threads)
    except OSError:
        pass
    # the GEMM alone on the dequantized operands: numpy binary64 and binary32 matmul (BLAS)
    # on 1024 activation rows against the whole weight, in TFLOP/s
    ca, sa, ga, _ = oracle.quantize(np.ascontiguousarray(x_np[:1024]), rht=True, rht_seed=W.RHT_SEED)
    cwt, swt, gw, _ = oracle.quantize(np.ascontiguousarray(w_np.T), blocking=oracle.BLOCK_16x16)
    a64 = oracle.block_values_f64(ca, sa, 1024, K, 0) * float(ga)
    b64 = oracle.block_values_f64(cwt, swt, NN, K, 1) * float(gw)
    fl = 2.0 * 1024 * NN * K
    for name, dt in (("gemm_f64_TFLOPs", np.float64), ("gemm_f32_TFLOPs", np.float32)):
        aa, bb = a64.astype(dt), np.ascontiguousarray(b64.T.astype(dt))
        np.matmul(aa[:64], bb)
        t0 = time.perf_counter()
        np.matmul(aa, bb)
        rates[name] = round(fl / (time.perf_counter() - t0) / 1e12, 4)
    del a64, b64
    what = ("the whole step (all %d activation rows)" % M if sample_rows == M else
            "%d of %d activation rows, scaled to one step" % (sample_rows, M))
    return {"value": round(flops / t_step / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model, "host_cpus": os.cpu_count(),
            "sample": "%s: quantize X (RHT, 1x16), quantize W and W^T (16x16), binary64 GEMM, "
                      "dequantize X; median of %d runs, %.1f s of CPU work in all"
                      % (what, repeats, work),
            "seconds_per_step_est": round(t_step, 2), **rates}


def _csv_rows(pattern_dir, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(pattern_dir, "**", "*" + suffix), recursive=True)):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _field(row, *names):
    for n in names:
        v = row.get(n)
        if v not in (None, ""):
            return v
    return None


def _short_name(name):
    """A kernel's name without the return type, namespaces and argument list."""
    name = name.replace("void ", "", 1).replace("(anonymous namespace)::", "")
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):   # the first '(' outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    return name[:cut].replace("nvfp4::", "")


def _kernel_key(row):
    name = _short_name(_field(row, "Kernel_Name") or "?")
    grid = int(_field(row, "Grid_Size_X", "Grid_Size") or 0)
    wg = int(_field(row, "Workgroup_Size_X", "Workgroup_Size") or 0)
    return name, grid, wg


def summarize(d, last=0):
    """Summary of a rocprofv3 ``--output-format csv`` directory.

    Kernel trace: per kernel and grid size, the dispatch durations in us (mean, median,
    p10, p90, min, max).  Counters: per kernel and grid size, the median over dispatches of
    each counter summed over its instances; FETCH_SIZE and WRITE_SIZE are also given in MB,
    scaled by what they read for the 256 MiB device copy of ``--copy-calibration`` when that
    copy is in the run.  ``last`` > 0 keeps only the last `last` dispatches of each kernel
    and grid, in dispatch order (the timed graph replay of a run with ``--steps last``)."""
    out = []
    trace = _csv_rows(d, "kernel_trace.csv")
    if trace:
        groups = {}
        for r in trace:
            t0, t1 = int(_field(r, "Start_Timestamp")), int(_field(r, "End_Timestamp"))
            groups.setdefault(_kernel_key(r), []).append((t0, (t1 - t0) / 1000.0))
        out.append("rocprofv3 kernel trace: durations in us%s" %
                   (", last %d dispatches of each kernel and grid" % last if last else ""))
        out.append("%-56s %9s %5s %6s %10s %10s %10s %10s %10s %10s" % (
            "kernel", "grid_thr", "wg", "calls", "mean", "median", "p10", "p90", "min", "max"))
        rows = []
        for (name, grid, wg), v in groups.items():
            v.sort()
            us = np.array([x[1] for x in v][-last:] if last else [x[1] for x in v])
            rows.append((us.sum(), name, grid, wg, us))
        for _, name, grid, wg, us in sorted(rows, key=lambda t: -t[0]):
            p10, med, p90 = np.percentile(us, [10, 50, 90])
            out.append("%-56s %9d %5d %6d %10.2f %10.2f %10.2f %10.2f %10.2f %10.2f" % (
                name[:56], grid, wg, us.size, us.mean(), med, p10, p90, us.min(), us.max()))
    ctr = _csv_rows(d, "counter_collection.csv")
    if ctr:
        per = {}   # (kernel key) -> dispatch -> counter -> summed value
        order = {}
        for r in ctr:
            key, disp = _kernel_key(r), int(_field(r, "Dispatch_Id", "Correlation_Id") or 0)
            cname = _field(r, "Counter_Name")
            per.setdefault(key, {}).setdefault(disp, {})
            per[key][disp][cname] = per[key][disp].get(cname, 0.0) + float(_field(r, "Counter_Value"))
        names = sorted({c for k in per.values() for dd in k.values() for c in dd})
        scale = {}
        copies = [(dd.get(c, 0.0), c) for (n, _, _), k in per.items() if "copyBuffer" in n
                  for dd in k.values() for c in ("FETCH_SIZE", "WRITE_SIZE")]
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            top = max([v for v, cc in copies if cc == c] or [0.0])
            if top > 100_000:   # only the 256 MiB calibration copy reaches 100 MB (KiB)
                scale[c] = (256 << 20) / 1024.0 / top
        out.append("")
        out.append("rocprofv3 counters: median per dispatch%s; counters summed over instances" %
                   (", last %d dispatches" % last if last else ""))
        for c, f in scale.items():
            out.append("calibration: %s counts %.4f of the bytes the 256 MiB copy moves "
                       "(scale x%.4f)" % (c, 1.0 / f, f))
        mfma = "SQ_VALU_MFMA_BUSY_CYCLES" in names and "GRBM_GUI_ACTIVE" in names
        if mfma:
            out.append("MFMA_busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 "
                       "XCDs); GRBM_GUI_ACTIVE also counts the window around a dispatch, so the "
                       "ratio means something for long dispatches only")
        hdr = "%-56s %9s %5s" % ("kernel", "grid_thr", "n")
        for c in names:
            hdr += " %16s" % c
            if c in scale:
                hdr += " %10s" % (c.split("_")[0].lower() + "_MB")
        if mfma:
            hdr += " %10s" % "MFMA_busy"
        out.append(hdr)
        for key in sorted(per, key=lambda k: k[0]):
            ds = [per[key][dd] for dd in sorted(per[key])]
            if last:
                ds = ds[-last:]
            line = "%-56s %9d %5d" % (key[0][:56], key[1], len(ds))
            meds = {}
            for c in names:
                med = meds[c] = float(np.median([dd.get(c, 0.0) for dd in ds]))
                line += " %16.6g" % med
                if c in scale:
                    line += " %10.2f" % (med * 1024.0 * scale[c] / 1e6)
            if mfma:
                cyc = 1024.0 * meds["GRBM_GUI_ACTIVE"] / 8.0
                line += " %9.1f%%" % (100.0 * meds["SQ_VALU_MFMA_BUSY_CYCLES"] / cyc if cyc else 0.0)
            out.append(line)
    if not out:
        out.append("no kernel_trace.csv or counter_collection.csv under %s" % d)
    return "\n".join(out)


def record_traffic(fetch_dir, write_dir, last=0):
    """HBM bytes of one workload-5 GEMM launch (the largest grid of gemm256_kernel<false>)
    from the FETCH_SIZE and WRITE_SIZE counter runs, each scaled by what it reads for the
    256 MiB calibration copy; written with the GEMM source's hash so that bench.py reports
    it only while the kernel is unchanged."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    res = {}
    for d, cname in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        per = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            if _field(r, "Counter_Name") != cname:
                continue
            key, disp = _kernel_key(r), int(_field(r, "Dispatch_Id", "Correlation_Id") or 0)
            per.setdefault(key, {}).setdefault(disp, 0.0)
            per[key][disp] += float(_field(r, "Counter_Value"))
        copy = max(v for (n, _, _), dd in per.items() if "copyBuffer" in n for v in dd.values())
        scale = (256 << 20) / 1024.0 / copy
        gkeys = [k for k in per if k[0].startswith("gemm256_kernel<false>")]
        gk = max(gkeys, key=lambda k: k[1])
        vals = [per[gk][dd] for dd in sorted(per[gk])]
        if last:
            vals = vals[-last:]
        res[cname] = (float(np.median(vals)) * 1024.0 * scale, scale, gk[0], len(vals))
    src = os.path.join(here, "block_scaled_fp4_06_amd", "csrc", "gemm.hip")
    rec = {"kernel": res["FETCH_SIZE"][2], "workload": "8192x20480x5120 bf16 out",
           "dispatches": res["FETCH_SIZE"][3],
           "read_bytes": res["FETCH_SIZE"][0], "write_bytes": res["WRITE_SIZE"][0],
           "fetch_scale": round(res["FETCH_SIZE"][1], 4), "write_scale": round(res["WRITE_SIZE"][1], 4),
           "source_sha256": hashlib.sha256(open(src, "rb").read()).hexdigest(),
           "commands": ["rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s -o bench -- python3 "
                        "bench.py --steps 2 --warmup 1 --no-cpu-baseline --copy-calibration"
                        % fetch_dir,
                        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s -o bench -- python3 "
                        "bench.py --steps 2 --warmup 1 --no-cpu-baseline --copy-calibration"
                        % write_dir],
           "traffic_bytes": res["FETCH_SIZE"][0] + res["WRITE_SIZE"][0]}
    path = os.path.join(here, "profiles", "gemm_w5_traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    return path


def graph_of(fn, calls):
    """A HIP graph of `calls` back-to-back invocations of fn (captured on a side stream)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        for _ in range(calls):
            fn()
    return g


def replay_ms(g, reps=1):
    """Event-timed milliseconds of `reps` replays of graph g on the current stream (the
    replay launches there), after one untimed replay."""
    import torch
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def main():
    args = parse()
    if args.summarize:
        print(summarize(args.summarize, args.last))
        return
    if args.record_traffic:
        print(record_traffic(*args.record_traffic, last=args.last))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    from block_scaled_fp4_06_amd import nvfp4 as N
    from block_scaled_fp4_06_amd import workloads as W
    N.load()
    log("generating inputs")
    x_np = W.w3()
    w_np = W.w5_weight()
    X = to_dev(x_np)
    Wd = to_dev(w_np)
    dev = X.device
    # workspaces made before any capture (a zero-fill recorded in a graph would rerun on
    # every replay); the two quantizations run in stream order and share one
    ws_q = N.new_workspace(dev)
    ws_g = N.new_gemm_workspace(dev)
    qx = N.quantize(X, rht=True, rht_seed=W.RHT_SEED, workspace=ws_q)
    qw = N.quantize(Wd, blocking="16x16", with_transpose=True, workspace=ws_q)
    qwt = qw.transposed()
    C = torch.empty((M, NN), dtype=torch.bfloat16, device="cuda")
    Xh = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()

    calls = {
        "quantize_x": lambda: N.quantize(X, rht=True, rht_seed=W.RHT_SEED, out=qx, workspace=ws_q),
        "quantize_w": lambda: N.quantize(Wd, blocking="16x16", with_transpose=True, out=qw,
                                         workspace=ws_q),
        "gemm": lambda: N.gemm(qx, qwt, out=C, workspace=ws_g),
        "dequantize_x": lambda: N.dequantize(qx, out=Xh),
    }

    def step():
        for fn in calls.values():
            fn()

    names = list(calls)
    flops = 2.0 * M * NN * K
    work = {"quantize_x": (quant_bytes(M, K, "1x16"), "GB/s"),
            "quantize_w": (quant_bytes(K, NN, "16x16", True), "GB/s"),
            "gemm": (flops, "TFLOP/s"),
            "dequantize_x": (dequant_bytes(M, K, "1x16"), "GB/s")}

    def figures(t_ms, name):
        by, unit = work[name]
        if unit == "GB/s":
            ach = by / (t_ms * 1e-3) / 1e9
            return {"ms": round(t_ms, 4), "GBps": round(ach, 1),
                    "frac_hbm": round(ach / HBM_PEAK_GBPS, 4), "bytes": by}
        ach = by / (t_ms * 1e-3) / 1e12
        return {"ms": round(t_ms, 4), "TFLOPs": round(ach, 1),
                "frac_mfma_f16": round(ach / MFMA_F16_PEAK_TFLOPS, 4),
                "frac_mfma_fp4_context": round(ach / MFMA_FP4_PEAK_TFLOPS, 4)}

    # each kernel alone: a graph of `steps` back-to-back launches on the same (cache-warm)
    # input, replayed once untimed and once timed
    alone = {}
    for name in names:
        alone[name] = figures(replay_ms(graph_of(calls[name], args.steps)) / args.steps, name)
    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: a graph of one step, replayed `steps` times back to back (timed
    # with events around the replays) gives ms_per_step; each kernel's in-step time comes
    # from events recorded between eager launches of `steps` more steps (the host enqueues
    # far ahead of a GPU whose steps take milliseconds, and ROCm does not allow timing
    # events inside a captured graph)
    log("timing %d steps (graph replay)" % args.steps)
    how = "events between eager launches of the step"
    g1 = graph_of(step, 1)
    ms = replay_ms(g1, args.steps) / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record()
        for j, name in enumerate(names):
            calls[name]()
            evs[i][j + 1].record()
    torch.cuda.synchronize()
    kern = {name: figures(sum(evs[i][j].elapsed_time(evs[i][j + 1])
                              for i in range(args.steps)) / args.steps, name)
            for j, name in enumerate(names)}
    for name in names:
        log("%s: %.4f ms in the step (%.4f ms alone)" % (name, kern[name]["ms"], alone[name]["ms"]))
    g = kern["gemm"]
    out = {
        "metric": METRIC, "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16 MFMA / f32 accumulate (NVFP4 operands); f32 quantize arithmetic",
        "data": "synthetic",
        "config": {"workload": "NVFP4 linear layer, workload 5: quantize X 8192x5120 (RHT16, "
                               "1x16, RNE) + quantize W 5120x20480 (16x16, W and W^T) + GEMM "
                               "8192x20480x5120 (fp32 acc, bf16 out) + dequantize X",
                   "M": M, "N": NN, "K": K},
        "roofline": {"bound": "mfma", "achieved": g["TFLOPs"], "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": g["frac_mfma_f16"],
                     "traffic": gemm_traffic_bytes(), "kernel": "gemm"},
        "kernels": kern,
        "kernel_timing": how,
        "kernels_alone": alone,
    }
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = src.numel()
        del src, dst
    if not args.no_micro:
        log("device copy reference")
        cg = copy_bandwidth()
        out["copy_GBps"] = cg
        log("standalone quantize workloads")
        out["quantize"] = micro_quantize(N, W, copy_gbps=cg)
        log("MXFP4 quantize and GEMM")
        out["mxfp4"] = micro_mxfp4(N, W, copy_gbps=cg)
        log("linear layer step (fwd + bwd)")
        out["linear_step"] = micro_linear(N, W)
    if args.context:
        a16 = torch.randn((M, K), dtype=torch.float16, device="cuda")
        b16 = torch.randn((NN, K), dtype=torch.float16, device="cuda")
        for _ in range(3):
            torch.matmul(a16, b16.T)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            torch.matmul(a16, b16.T)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 10
        out["context_torch_f16_matmul_TFLOPs"] = round(flops / (t * 1e-3) / 1e12, 1)
        del a16, b16
        out["context_torch_mxfp4_scaled_mm_TFLOPs"] = context_scaled_mm_mx(N, W)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle, bounded sample)")
        out["cpu_baseline"] = cpu_baseline(x_np, w_np)
    torch.cuda.synchronize()   # nothing of ours is in flight when the process exits
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
