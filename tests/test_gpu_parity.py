"""GPU parity: libnvfp4's HIP kernels against the CPU oracle, through the C ABI.

Codes, scales and the tensor scale must be bit-exact; dequantized values bit-exact; the
GEMM within the stated tolerance of the binary64 reference.  Inputs are the seeded
workloads of block_scaled_fp4_06_amd.workloads at their full sizes, plus small and
ragged shapes and the degenerate cases.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from block_scaled_fp4_06_amd import nvfp4 as N  # noqa: E402
from block_scaled_fp4_06_amd import workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu

BLK = {"1x16": 0, "16x16": 1}
RND = {"rne": 0, "sr": 1}


def say(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.load()  # raises if libnvfp4.so is missing: no other implementation exists
    yield


def to_dev(x_u16: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(x_u16).view(np.int16)).view(torch.bfloat16).cuda()


def host(t):
    return t.cpu().numpy()


def run_quant(x_u16, blocking="1x16", rounding="rne", rht=False, rht_seed=0, sr_seed=0,
              sr_index_base=0, with_transpose=False, xdev=None):
    xd = to_dev(x_u16) if xdev is None else xdev
    q = N.quantize(xd, blocking=blocking, rounding=rounding, rht=rht, rht_seed=rht_seed,
                   sr_seed=sr_seed, sr_index_base=sr_index_base, with_transpose=with_transpose)
    torch.cuda.synchronize()
    return q


def oracle_quant(x_u16, blocking="1x16", rounding="rne", rht=False, rht_seed=0, sr_seed=0,
                 sr_index_base=0):
    return oracle.quantize(x_u16, blocking=BLK[blocking], rounding=RND[rounding], rht=rht,
                           rht_seed=rht_seed, sr_seed=sr_seed, sr_index_base=sr_index_base)


def assert_same(q, ref, check_codes=True):
    codes, scales, g, st = ref
    assert int(host(q.status)[0]) == st
    gd = host(q.global_dec)[0]
    if np.isnan(g):
        assert np.isnan(gd)
        return
    assert gd.view(np.uint32) == np.float32(g).view(np.uint32)
    assert np.array_equal(host(q.scales), scales)
    if check_codes:
        got = host(q.codes)
        if not np.array_equal(got, codes):
            bad = np.argwhere(got != codes)
            raise AssertionError("%d code bytes differ, first at %s: gpu %02x oracle %02x" % (
                len(bad), bad[0], got[tuple(bad[0])], codes[tuple(bad[0])]))


CASES = [
    # (rows, cols, blocking, rounding, rht)
    (16, 16, "1x16", "rne", False),
    (16, 16, "16x16", "rne", False),
    (48, 80, "1x16", "rne", True),
    (48, 80, "1x16", "sr", True),
    (48, 80, "16x16", "sr", False),
    (272, 528, "1x16", "rne", False),
    (272, 528, "1x16", "sr", False),
    (272, 528, "16x16", "rne", False),
    (1040, 2064, "1x16", "rne", True),
    (1040, 2064, "16x16", "sr", False),
    # RHT with 16x16 blocks (the transform runs along each row group first)
    (48, 80, "16x16", "rne", True),
    (272, 528, "16x16", "sr", True),
    (1040, 2064, "16x16", "rne", True),
]


@pytest.mark.parametrize("rows,cols,blocking,rounding,rht", CASES)
def test_quantize_small_shapes(rows, cols, blocking, rounding, rht):
    say("quantize %dx%d %s %s rht=%s" % (rows, cols, blocking, rounding, rht))
    x = W.normal_outliers(rows, cols, seed=rows * 7 + cols)
    kw = dict(blocking=blocking, rounding=rounding, rht=rht, rht_seed=0x1234, sr_seed=99)
    assert_same(run_quant(x, **kw), oracle_quant(x, **kw))


def test_quantize_row_stride():
    say("quantize with ld != cols")
    big = W.normal_outliers(64, 256, seed=5)
    view = to_dev(big)[:, 32:32 + 160]
    x = np.ascontiguousarray(big[:, 32:32 + 160])
    for kw in (dict(rht=True, rht_seed=3), dict(rounding="sr", sr_seed=5),
               dict(blocking="16x16", rounding="sr", sr_seed=6)):
        assert_same(run_quant(None, xdev=view, **kw), oracle_quant(x, **kw))
    # 16x16 with the W^T output, with and without the transform: W^T's codes and scales
    # are the transposes of W's
    for kw in (dict(blocking="16x16"), dict(blocking="16x16", rht=True, rht_seed=4)):
        q = run_quant(None, xdev=view, with_transpose=True, **kw)
        ref = oracle_quant(x, **kw)
        assert_same(q, ref)
        full = np.empty((64, 160), np.uint8)
        full[:, 0::2], full[:, 1::2] = ref[0] & 0xF, ref[0] >> 4
        ft = np.ascontiguousarray(full.T)
        assert np.array_equal(host(q.codes_t), (ft[:, 0::2] | (ft[:, 1::2] << 4)).astype(np.uint8))
        assert np.array_equal(host(q.scales_t), np.ascontiguousarray(ref[1].T))


def test_w1_full():
    say("workload 1: 256x256 1x16 RNE")
    x = W.w1()
    ref = oracle_quant(x)
    q = run_quant(x)
    assert_same(q, ref)
    # dequantize (fp32 and bf16) bit-exact, and the per-block max error report
    y32 = N.dequantize(q, torch.float32)
    yb = N.dequantize(q, torch.bfloat16)
    torch.cuda.synchronize()
    r32 = oracle.dequantize(ref[0], ref[1], ref[2], 256, 256)
    assert np.array_equal(host(y32).view(np.uint32), r32.view(np.uint32))
    rb = oracle.dequantize_bf16(ref[0], ref[1], ref[2], 256, 256)
    assert np.array_equal(host(yb.view(torch.int16)).view(np.uint16), rb)
    err = np.abs(host(y32) - W.bf16_bits_to_f32(x)).reshape(256, 16, 16).max(axis=2)
    say("w1 per-block max |x - xhat|: max %.4g median %.4g" % (err.max(), np.median(err)))


def test_w2_full_and_transpose():
    say("workload 2: 4096x4096 16x16 RNE, W and W^T")
    x = W.w2()
    ref = oracle_quant(x, blocking="16x16")
    q = run_quant(x, blocking="16x16", with_transpose=True)
    assert_same(q, ref)
    xt = np.ascontiguousarray(x.T)
    ref_t = oracle_quant(xt, blocking="16x16")
    assert np.array_equal(host(q.codes_t), ref_t[0])
    assert np.array_equal(host(q.scales_t), ref_t[1])
    qt = run_quant(xt, blocking="16x16")
    assert_same(qt, ref_t)


def test_w3_full():
    say("workload 3: 8192x5120 RHT + 1x16 RNE")
    x = W.w3()
    kw = dict(rht=True, rht_seed=W.RHT_SEED)
    assert_same(run_quant(x, **kw), oracle_quant(x, **kw))




def test_w5_weight_full():
    say("workload 5 weight: 5120x20480 16x16 RNE with W^T")
    x = W.w5_weight()
    ref = oracle_quant(x, blocking="16x16")
    q = run_quant(x, blocking="16x16", with_transpose=True)
    assert_same(q, ref)
    c = ref[0]
    lo, hi = c & 0xF, c >> 4
    full = np.empty((c.shape[0], c.shape[1] * 2), np.uint8)
    full[:, 0::2], full[:, 1::2] = lo, hi
    ft = np.ascontiguousarray(full.T)
    packed_t = (ft[:, 0::2] | (ft[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(host(q.codes_t), packed_t)
    assert np.array_equal(host(q.scales_t), ref[1].T)


def test_more_chunks_than_resident_workgroups():
    # 8192 x 8192 with RHT: 4.2M row groups, more 1x16 chunks than the GPU holds in
    # registers, so some workgroups re-read the chunks they could not keep
    say("1x16 RHT RNE 8192x8192: chunks re-read after the tensor scale")
    x = W.normal_outliers(8192, 8192, seed=11)
    kw = dict(rht=True, rht_seed=W.RHT_SEED)
    assert_same(run_quant(x, **kw), oracle_quant(x, **kw))


@pytest.fixture
def help_at_once(monkeypatch):
    # every waiting workgroup computes the partial maxima it has not seen yet itself
    monkeypatch.setenv("NVFP4_HELP_DELAY_TICKS", "0")
    yield


def test_waiters_compute_missing_partials(help_at_once):
    say("help path: waiters compute missing partial maxima themselves")
    x = W.normal_outliers(2048, 5120, seed=12)
    for kw in (dict(rht=True, rht_seed=3), dict()):
        assert_same(run_quant(x, **kw), oracle_quant(x, **kw))
    w = W.normal_scaled(2048, 1024, seed=13, std=0.02)
    ref = oracle_quant(w, blocking="16x16")
    q = run_quant(w, blocking="16x16", with_transpose=True)
    assert_same(q, ref)
    ref_t = oracle_quant(np.ascontiguousarray(w.T), blocking="16x16")
    assert np.array_equal(host(q.codes_t), ref_t[0])
    assert np.array_equal(host(q.scales_t), ref_t[1])
    kw = dict(blocking="16x16", rht=True, rht_seed=9)
    assert_same(run_quant(w, **kw), oracle_quant(w, **kw))


def test_graph_replay():
    # a captured quantize replayed on new data: every launch must tag its workspace state
    # afresh, or a replay could take the previous replay's partial maxima for its own
    say("HIP graph replay of quantize (1x16 RHT, 16x16 with W^T) on changing inputs")
    xs = [W.normal_outliers(1024, 2048, seed=s) for s in (21, 22, 23)]
    xs[1] = W.normal_scaled(1024, 2048, seed=24, std=0.001)   # a much smaller tensor amax
    for kw in (dict(rht=True, rht_seed=5), dict(blocking="16x16", with_transpose=True)):
        xd = to_dev(xs[0])
        ws = N.new_workspace(xd.device)
        q = N.quantize(xd, workspace=ws, **kw)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=side):
            N.quantize(xd, out=q, workspace=ws, **kw)
        torch.cuda.synchronize()
        okw = {k: v for k, v in kw.items() if k != "with_transpose"}
        for i in (1, 0, 2, 1, 1, 0):
            xd.copy_(to_dev(xs[i]))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert_same(q, oracle_quant(xs[i], **okw))
            # eager work on the same workspace between replays
            N.quantize(xd, out=q, workspace=ws, **kw)
            torch.cuda.synchronize()
            assert_same(q, oracle_quant(xs[i], **okw))


def test_w5_weight_rht_full():
    # the weight transformed along K with the activations' sign vector (16x16 blocks, W^T
    # emitted alongside): both GEMM operands carry the same transform
    say("workload 5 weight, RHT along K + 16x16 RNE, with its transpose")
    wt = np.ascontiguousarray(W.w5_weight().T)     # 20480 x 5120, K contiguous
    kw = dict(blocking="16x16", rht=True, rht_seed=W.RHT_SEED)
    ref = oracle_quant(wt, **kw)
    q = run_quant(wt, with_transpose=True, **kw)
    assert_same(q, ref)
    c = ref[0]
    full = np.empty((c.shape[0], c.shape[1] * 2), np.uint8)
    full[:, 0::2], full[:, 1::2] = c & 0xF, c >> 4
    ft = np.ascontiguousarray(full.T)
    assert np.array_equal(host(q.codes_t), (ft[:, 0::2] | (ft[:, 1::2] << 4)).astype(np.uint8))
    assert np.array_equal(host(q.scales_t), ref[1].T)


def test_gemm_both_operands_transformed():
    # X W with the same RHT on the K-groups of both operands: the GEMM kernel is the same;
    # parity against the oracle, and the product approximates the untransformed one
    say("GEMM with RHT on both operands (16x16 weight)")
    M, N_, K = 512, 768, 1024
    x = W.channel_outliers(M, K, seed=41)
    w = W.normal_scaled(K, N_, seed=42, std=0.02)
    wt = np.ascontiguousarray(w.T)
    ka = dict(rht=True, rht_seed=W.RHT_SEED)
    kb = dict(blocking="16x16", rht=True, rht_seed=W.RHT_SEED)
    qa, qb = run_quant(x, **ka), run_quant(wt, **kb)
    ra, rb = oracle_quant(x, **ka), oracle_quant(wt, **kb)
    assert_same(qa, ra)
    assert_same(qb, rb)
    gemm_check(qa, qb, ra, rb, M, N_, K)
    c = host(N.gemm(qa, qb, torch.float32)).astype(np.float64)
    exact = W.bf16_bits_to_f32(x).astype(np.float64) @ W.bf16_bits_to_f32(w).astype(np.float64)
    assert np.linalg.norm(c - exact) / np.linalg.norm(exact) < 0.2


@pytest.mark.parametrize("name", ["w2", "w5_weight"])
def test_weight_granularity_study(name):
    # 1x16 against 16x16 blocks on the weights, through the GPU quantize and dequantize;
    # the dequantized values are the oracle's bit for bit, so the errors are too
    x = W.w2() if name == "w2" else W.w5_weight()
    rows, cols = x.shape
    xd = to_dev(x)
    xf = torch.from_numpy(W.bf16_bits_to_f32(x)).cuda().double()
    out = {}
    for blk in ("1x16", "16x16"):
        q = run_quant(x, blocking=blk, xdev=xd)
        y = N.dequantize(q, torch.float32).double()
        d = y - xf
        out[blk] = (float(d.norm() / xf.norm()), float(d.abs().max()))
        if name == "w2":
            ref = oracle.dequantize(*oracle_quant(x, blocking=blk)[:3], rows, cols, BLK[blk])
            assert np.array_equal(host(y.float()).view(np.uint32), ref.view(np.uint32))
    say("granularity %s: rel-fro 1x16 %.4f 16x16 %.4f | max abs 1x16 %.3g 16x16 %.3g" % (
        name, out["1x16"][0], out["16x16"][0], out["1x16"][1], out["16x16"][1]))
    assert out["16x16"][0] > out["1x16"][0]


def test_edge_values():
    say("edge values: zeros, -0, subnormal, huge, non-finite")
    z = np.zeros((32, 64), np.uint16)
    assert_same(run_quant(z), oracle_quant(z))
    assert_same(run_quant(z, rht=True, rht_seed=1), oracle_quant(z, rht=True, rht_seed=1))
    negz = np.full((32, 64), 0x8000, np.uint16)
    assert_same(run_quant(negz, rounding="sr"), oracle_quant(negz, rounding="sr"))
    rng = np.random.default_rng(0)
    sub = rng.integers(0, 0x80, (64, 64)).astype(np.uint16) | (rng.integers(0, 2, (64, 64)).astype(np.uint16) << 15)
    for kw in (dict(), dict(rht=True, rht_seed=9), dict(rounding="sr", sr_seed=4),
               dict(blocking="16x16")):
        assert_same(run_quant(sub, **kw), oracle_quant(sub, **kw))
    huge = W.normal_outliers(64, 64, seed=1)
    huge[5, 7] = 0x7F7F   # largest finite bf16
    for kw in (dict(), dict(rht=True, rht_seed=2), dict(rounding="sr", sr_seed=1)):
        assert_same(run_quant(huge, **kw), oracle_quant(huge, **kw))
    tiny_amax = np.zeros((16, 32), np.uint16)
    tiny_amax[3, 3] = 0x0001  # one subnormal element: s_enc overflows and is clamped
    tiny_amax[9, 30] = 0x8001
    for kw in (dict(), dict(rounding="sr"), dict(blocking="16x16")):
        assert_same(run_quant(tiny_amax, **kw), oracle_quant(tiny_amax, **kw))
    # RHT with a tensor scale too large for the folded quarter (the multiplier table
    # exceeds 2^108): the kernels scale every transformed value by 1/4 first
    for kw in (dict(rht=True, rht_seed=5), dict(rht=True, rht_seed=5, rounding="sr", sr_seed=2)):
        assert_same(run_quant(tiny_amax, **kw), oracle_quant(tiny_amax, **kw))
    small = W.f32_to_bf16_bits(rng.standard_normal((64, 64)).astype(np.float32) * np.float32(1e-30))
    pick = rng.random((64, 64)) < 0.3
    small[pick] = sub[pick]
    # normal-range tensor with bf16 subnormals inside its row groups: folded quarter,
    # tiny transformed values round to zero codes with their sign
    mixed = W.normal_outliers(64, 64, seed=6)
    pick = rng.random((64, 64)) < 0.3
    mixed[pick] = sub[pick]
    for xin in (small, mixed):
        for kw in (dict(rht=True, rht_seed=6), dict(rht=True, rht_seed=6, rounding="sr", sr_seed=3),
                   dict(rht=True, rht_seed=6, blocking="16x16")):
            assert_same(run_quant(xin, **kw), oracle_quant(xin, **kw))
    for bad in (0x7F80, 0xFF80, 0x7FC1):
        x = W.normal_outliers(32, 32, seed=3)
        x[7, 9] = bad
        for kw in (dict(), dict(rht=True, rht_seed=3), dict(blocking="16x16")):
            assert_same(run_quant(x, **kw), oracle_quant(x, **kw), check_codes=False)


def test_empty_tensor():
    say("empty tensor")
    x = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    q = N.quantize(x)
    torch.cuda.synchronize()
    assert host(q.global_dec)[0] == 1.0 and int(host(q.status)[0]) == 0


def test_determinism_and_chunking():
    say("determinism and sr_index_base chunking")
    x = W.w4(512, 1024).copy()
    x[0, 0] = 0x4200
    x[256, 0] = 0x4200   # both halves hold the tensor amax
    kw = dict(rounding="sr", sr_seed=17)
    a = run_quant(x, **kw)
    b = run_quant(x, **kw)
    assert np.array_equal(host(a.codes), host(b.codes))
    xd = to_dev(x)
    h0 = run_quant(None, xdev=xd[:256], **kw)
    h1 = run_quant(None, xdev=xd[256:], sr_index_base=256 * 1024, **kw)
    assert np.array_equal(np.concatenate([host(h0.codes), host(h1.codes)]), host(a.codes))
    assert_same(a, oracle_quant(x, **kw))


@pytest.mark.parametrize("blocking", ["1x16", "16x16"])
def test_dequantize_parity(blocking):
    say("dequantize %s" % blocking)
    x = W.normal_outliers(272, 528, seed=11)
    ref = oracle_quant(x, blocking=blocking)
    q = run_quant(x, blocking=blocking)
    r32 = oracle.dequantize(ref[0], ref[1], ref[2], 272, 528, BLK[blocking])
    rb = oracle.dequantize_bf16(ref[0], ref[1], ref[2], 272, 528, BLK[blocking])
    y32 = N.dequantize(q, torch.float32)
    out = torch.full((272, 544), -1.0, dtype=torch.bfloat16, device="cuda")
    yb = N.dequantize(q, torch.bfloat16, out=out[:, :528])
    torch.cuda.synchronize()
    assert np.array_equal(host(y32).view(np.uint32), r32.view(np.uint32))
    assert np.array_equal(host(yb.view(torch.int16)).view(np.uint16), rb)
    assert torch.all(out[:, 528:] == -1.0)   # the row stride is honoured


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_dequantize_output_beyond_2gib(out_dtype):
    """Outputs past 2 GiB (64-bit element offsets): 32768 x 32768 elements (4 GiB of fp32,
    2 GiB of bf16) from random codes and E4M3 scales, sampled 16-row slices (the last
    included) against the oracle."""
    rows = cols = 32768
    say("dequantize %dx%d to %s" % (rows, cols, out_dtype))
    g = torch.Generator(device="cuda").manual_seed(23)
    codes = torch.randint(0, 256, (rows, cols // 2), dtype=torch.uint8, device="cuda", generator=g)
    scales = torch.randint(0, 0x7F, (rows, cols // 16), dtype=torch.uint8, device="cuda", generator=g)
    gd = torch.tensor([0.375], dtype=torch.float32, device="cuda")
    q = N.NVFP4Tensor(codes, scales, gd, rows, cols, N.BLOCK_1x16)
    f32 = out_dtype == "f32"
    y = N.dequantize(q, torch.float32 if f32 else torch.bfloat16)
    torch.cuda.synchronize()
    for r in (0, 12336, rows // 2, rows - 16):   # 16-row slices (the oracle's row unit)
        c = host(codes[r:r + 16])
        sc = host(scales[r:r + 16])
        if f32:
            ref = oracle.dequantize(c, sc, np.float32(0.375), 16, cols)
            assert np.array_equal(host(y[r:r + 16]).view(np.uint32), ref.view(np.uint32)), r
        else:
            ref = oracle.dequantize_bf16(c, sc, np.float32(0.375), 16, cols)
            assert np.array_equal(host(y[r:r + 16].view(torch.int16)).view(np.uint16), ref), r
    del y, codes, scales
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- GEMM
def gemm_check(qa, qb, ref_a, ref_b, M, N_, K, rows=None):
    """Two-part gate: fp32 output within 1e-3 relative Frobenius of the binary64 product
    (plus the per-element fp32 summation bound), and bf16 output within 1e-3 of the
    bf16-rounded binary64 product."""
    c32 = N.gemm(qa, qb, torch.float32)
    cb = N.gemm(qa, qb, torch.bfloat16)
    torch.cuda.synchronize()
    a_t = (ref_a[0], ref_a[1], ref_a[2], M, K, qa.blocking)
    b_t = (ref_b[0], ref_b[1], ref_b[2], N_, K, qb.blocking)
    sl = rows if rows is not None else slice(None)
    cref = oracle.gemm_reference(a_t, b_t, row_slice=sl)
    g32 = host(c32)[sl].astype(np.float64)
    gb = W.bf16_bits_to_f32(host(cb.view(torch.int16)).view(np.uint16)[sl]).astype(np.float64)
    fro = np.linalg.norm(cref)
    e32 = np.linalg.norm(g32 - cref) / max(fro, 1e-300)
    cref_bf16 = W.bf16_bits_to_f32(W.f32_to_bf16_bits(cref.astype(np.float32))).astype(np.float64)
    eb = np.linalg.norm(gb - cref_bf16) / max(np.linalg.norm(cref_bf16), 1e-300)
    eb_raw = np.linalg.norm(gb - cref) / max(fro, 1e-300)
    say("gemm %dx%dx%d: rel-fro fp32 %.3g, bf16 vs bf16(ref) %.3g, bf16 vs ref %.3g" % (
        M, N_, K, e32, eb, eb_raw))
    assert e32 <= 1e-3
    assert eb <= 1e-3
    # per element: |fl(sum) - sum| <= gamma_K * sum |a||b| (K u / (1 - K u)), plus the
    # epilogue's two roundings
    qa64 = oracle.block_values_f64(*a_t[:2], M, K, qa.blocking)[sl]
    qb64 = oracle.block_values_f64(*b_t[:2], N_, K, qb.blocking)
    absprod = np.abs(qa64) @ np.abs(qb64).T * float(ref_a[2]) * float(ref_b[2])
    u = 2.0 ** -24
    bound = (K * u / (1 - K * u) + 3 * u) * absprod + 1e-37
    assert np.all(np.abs(g32 - cref) <= bound)
    return e32, eb


GEMM_SHAPES = [(128, 128, 64), (144, 208, 80), (256, 384, 320), (48, 16, 16), (16, 48, 528),
               (400, 272, 1056),
               # K % 256 == 0: the 256 x 256-tile kernel, with ragged M and N
               (256, 256, 256), (400, 272, 1024), (48, 16, 512), (1040, 784, 2304)]


@pytest.mark.parametrize("M,N_,K", GEMM_SHAPES)
def test_gemm_small(M, N_, K):
    say("gemm %dx%dx%d" % (M, N_, K))
    a = W.channel_outliers(M, K, seed=M + K)
    w = W.normal_scaled(K, N_, seed=N_ + K, std=0.02)   # K x N weight
    ka = dict(rht=True, rht_seed=W.RHT_SEED)
    qa = run_quant(a, **ka)
    qw = run_quant(w, blocking="16x16", with_transpose=True)
    ref_a = oracle_quant(a, **ka)
    wt = np.ascontiguousarray(w.T)
    ref_b = oracle_quant(wt, blocking="16x16")
    qb = qw.transposed()
    assert np.array_equal(host(qb.codes), ref_b[0])
    gemm_check(qa, qb, ref_a, ref_b, M, N_, K)


def test_gemm_other_blockings():
    say("gemm A 16x16, B 1x16 with SR")
    M, N_, K = 96, 160, 192
    a = W.normal_scaled(M, K, seed=1, std=1.0)
    b = W.w4(N_, K)
    qa, ra = run_quant(a, blocking="16x16"), oracle_quant(a, blocking="16x16")
    kb = dict(rounding="sr", sr_seed=3, rht=True, rht_seed=8)
    qb, rb = run_quant(b, **kb), oracle_quant(b, **kb)
    gemm_check(qa, qb, ra, rb, M, N_, K)


def gemm_check_all_rows(qa, qb, ref_a, ref_b, M, N_, K, chunk=512):
    """gemm_check's two-part gate and per-element bound on every row of C, in row chunks of
    the binary64 reference (its full C would take 1.3 GB per copy at workload-5 size)."""
    c32 = N.gemm(qa, qb, torch.float32)
    cb = N.gemm(qa, qb, torch.bfloat16)
    torch.cuda.synchronize()
    a_t = (ref_a[0], ref_a[1], ref_a[2], M, K, qa.blocking)
    b_t = (ref_b[0], ref_b[1], ref_b[2], N_, K, qb.blocking)
    err32 = ref2 = errb = refb2 = 0.0
    u = 2.0 ** -24
    for r0, r1, cref, absprod in oracle.gemm_reference_chunks(a_t, b_t, chunk, with_abs=True):
        g32 = host(c32[r0:r1]).astype(np.float64)
        gb = W.bf16_bits_to_f32(host(cb[r0:r1].view(torch.int16)).view(np.uint16)).astype(np.float64)
        cref_bf16 = W.bf16_bits_to_f32(W.f32_to_bf16_bits(cref.astype(np.float32))).astype(np.float64)
        err32 += float(np.sum((g32 - cref) ** 2))
        ref2 += float(np.sum(cref ** 2))
        errb += float(np.sum((gb - cref_bf16) ** 2))
        refb2 += float(np.sum(cref_bf16 ** 2))
        bound = (K * u / (1 - K * u) + 3 * u) * absprod + 1e-37
        bad = np.argwhere(np.abs(g32 - cref) > bound)
        assert bad.size == 0, "row %d col %d outside the fp32 summation bound" % (
            r0 + bad[0][0], bad[0][1])
        if r0 % 2048 == 0:
            say("gemm rows %d..%d checked" % (r0, r1))
    e32 = np.sqrt(err32) / max(np.sqrt(ref2), 1e-300)
    eb = np.sqrt(errb) / max(np.sqrt(refb2), 1e-300)
    say("gemm %dx%dx%d, all rows: rel-fro fp32 %.3g, bf16 vs bf16(ref) %.3g" % (M, N_, K, e32, eb))
    assert e32 <= 1e-3
    assert eb <= 1e-3
    return e32, eb


def test_gemm_w5_full_all_rows():
    say("workload 5: 8192x5120 . (5120x20480) GEMM, every row")
    a = W.w3()
    w = W.w5_weight()
    ka = dict(rht=True, rht_seed=W.RHT_SEED)
    qa = run_quant(a, **ka)
    qw = run_quant(w, blocking="16x16", with_transpose=True)
    ref_a = oracle_quant(a, **ka)
    assert_same(qa, ref_a)
    ref_w = oracle_quant(w, blocking="16x16")
    c = ref_w[0]
    full = np.empty((c.shape[0], c.shape[1] * 2), np.uint8)
    full[:, 0::2], full[:, 1::2] = c & 0xF, c >> 4
    ft = np.ascontiguousarray(full.T)
    ref_b = ((ft[:, 0::2] | (ft[:, 1::2] << 4)).astype(np.uint8),
             np.ascontiguousarray(ref_w[1].T), ref_w[2], 0)
    del full, ft
    gemm_check_all_rows(qa, qw.transposed(), ref_a, ref_b, 8192, 20480, 5120)


def spread_blocks(x_bits, seed, octaves=12):
    """bf16 input whose 16-element row groups are scaled by 2^-j, j uniform in 0..octaves:
    block scales then span ~2^12, so fp32 sums of the products round."""
    rng = np.random.default_rng(seed)
    f = W.bf16_bits_to_f32(x_bits).reshape(x_bits.shape[0], -1, 16)
    f = f * np.exp2(-rng.integers(0, octaves + 1, size=f.shape[:2] + (1,))).astype(np.float32)
    return W.f32_to_bf16_bits(f.reshape(x_bits.shape).astype(np.float32))


@pytest.mark.parametrize("M,N_,K,spread", [(4096, 5120, 8192, False), (528, 800, 8192, False),
                                           (256, 256, 32768, False), (528, 800, 8192, True),
                                           (256, 256, 32768, True)])
def test_gemm_split_tail(M, N_, K, spread):
    # nvfp4_gemm_ws splits the tiles of the last, partial round along K, each split keeping
    # at least 8 K steps (4096 x 5120: 256 whole tiles, then 64 tiles in 4 K ranges;
    # 528 x 800: 12 edge-heavy tiles in 4; 256 x 256: one tile in 8): against the oracle
    # on rows of both kinds of tiles, against the unsplit kernel, bit-identical from run to
    # run, counters back at zero.  On the plain workloads every fp32 partial sum is exact
    # (the products sit on a coarse grid: block scales within a few octaves), so split and
    # unsplit agree bit for bit; with block magnitudes spread over 12 octaves the sums
    # round and the two differ within the fp32 summation bound.
    say("gemm split tail %dx%dx%d%s" % (M, N_, K, " (spread blocks)" if spread else ""))
    a = W.channel_outliers(M, K, seed=M + 3)
    if spread:
        a = spread_blocks(a, seed=M)
    w = W.normal_scaled(K, N_, seed=N_ + 4, std=0.02)
    ka = dict(rht=True, rht_seed=W.RHT_SEED)
    qa, ref_a = run_quant(a, **ka), oracle_quant(a, **ka)
    qw = run_quant(w, blocking="16x16", with_transpose=True)
    qb = qw.transposed()
    ref_b = oracle_quant(np.ascontiguousarray(w.T), blocking="16x16")
    assert np.array_equal(host(qb.codes), ref_b[0])
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([rng.choice(M, 24, replace=False), [0, M - 1],
                                     rng.choice(np.arange(M - M // 4, M), 16, replace=False)]))
    gemm_check(qa, qb, ref_a, ref_b, M, N_, K, rows=rows)
    ws = N.new_gemm_workspace(qa.codes.device)
    c1 = N.gemm(qa, qb, torch.float32, workspace=ws)
    c2 = N.gemm(qa, qb, torch.float32, workspace=ws)
    c0 = N.gemm(qa, qb, torch.float32, split_tail=False)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    assert int(ws[:4096].count_nonzero()) == 0
    assert int(ws[4096:].count_nonzero()) > 0       # the split path ran: partial tiles
    d = float((c1.double() - c0.double()).norm() / c0.double().norm())
    say("  split vs unsplit: rel-fro %.3g, %d elements differ" % (d, int((c1 != c0).sum())))
    assert d <= 1e-5
    qa64 = oracle.block_values_f64(ref_a[0], ref_a[1], M, K, 0)[rows] * float(ref_a[2])
    qb64 = oracle.block_values_f64(ref_b[0], ref_b[1], N_, K, 1) * float(ref_b[2])
    u = 2.0 ** -24
    bound = 2 * (K * u / (1 - K * u) + 3 * u) * (np.abs(qa64) @ np.abs(qb64).T) + 1e-37
    diff = np.abs(host(c1)[rows].astype(np.float64) - host(c0)[rows].astype(np.float64))
    assert np.all(diff <= bound)


def test_gemm_split_tail_strided_output():
    # the last split item writes through the same epilogue: a row stride wider than N
    # (both output types), padding columns untouched
    say("gemm split tail into a strided C (ldc 832 > N 800)")
    M, N_, K = 528, 800, 8192
    qa = run_quant(W.channel_outliers(M, K, seed=41), rht=True, rht_seed=W.RHT_SEED)
    qb = run_quant(W.normal_scaled(K, N_, seed=42, std=0.02), blocking="16x16",
                   with_transpose=True).transposed()
    for dt in (torch.float32, torch.bfloat16):
        ref = N.gemm(qa, qb, dt)
        big = torch.zeros((M, 832), dtype=dt, device=ref.device)
        N.gemm(qa, qb, out=big[:, :N_])
        torch.cuda.synchronize()
        assert torch.equal(big[:, :N_], ref)
        assert int(big[:, N_:].count_nonzero()) == 0


def test_gemm_split_tail_graph_replay():
    # counters reset by the last arrival of every launch: a captured split GEMM replayed on
    # changing operands, with eager calls on the same workspace in between
    say("HIP graph replay of a split GEMM (12 tiles x 4 K ranges) on changing inputs")
    M, N_, K = 528, 800, 8192
    ka = dict(rht=True, rht_seed=W.RHT_SEED)
    ins = []
    for sd in (31, 32, 33):
        a = W.channel_outliers(M, K, seed=sd)
        w = W.normal_scaled(K, N_, seed=sd + 10, std=0.02)
        ins.append((run_quant(a, **ka), run_quant(w, blocking="16x16", with_transpose=True).transposed()))
    qa, qb = run_quant(W.channel_outliers(M, K, seed=30), **ka), ins[0][1]
    qb = N.NVFP4Tensor(qb.codes.clone(), qb.scales.clone(), qb.global_dec.clone(), qb.rows,
                       qb.cols, qb.blocking)
    ws = N.new_gemm_workspace(qa.codes.device)
    out = torch.empty((M, N_), dtype=torch.float32, device=qa.codes.device)
    N.gemm(qa, qb, out=out, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        N.gemm(qa, qb, out=out, workspace=ws, stream=side)
    torch.cuda.synchronize()
    for i in (1, 0, 2, 2, 1):
        xa, xb = ins[i]
        for dst, src in ((qa.codes, xa.codes), (qa.scales, xa.scales), (qa.global_dec, xa.global_dec),
                         (qb.codes, xb.codes), (qb.scales, xb.scales), (qb.global_dec, xb.global_dec)):
            dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = N.gemm(xa, xb, torch.float32, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        assert int(ws[:4096].count_nonzero()) == 0


def test_gemm_operand_beyond_2gib():
    # A of 524800 x 8192 (2.15 GB of codes): rows past the 2^31-byte mark must be read,
    # not returned as zero by a clamped buffer range.  Codes and E4M3 scales are drawn
    # directly (the GEMM is defined on any operand); sampled rows on both sides of the
    # mark are checked against the oracle's binary64 product.
    say("gemm with a 2.15 GB operand (524800 x 8192 codes)")
    M, N_, K = 524800, 256, 8192
    g = torch.Generator(device="cuda").manual_seed(1)
    ac = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    asc = torch.randint(0x28, 0x48, (M, K // 16), dtype=torch.uint8, device="cuda", generator=g)
    bc = torch.randint(0, 256, (N_, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    bsc = torch.randint(0x28, 0x48, (N_, K // 16), dtype=torch.uint8, device="cuda", generator=g)
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    qa = N.NVFP4Tensor(ac, asc, one, M, K, 0)
    qb = N.NVFP4Tensor(bc, bsc, one, N_, K, 0)
    c = N.gemm(qa, qb, torch.float32)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 131071, 262143, 262144, 393216, 524286, 524287, 524288, 524289,
                     524290, 524543, 524544, 524700, M - 2, M - 1])   # 16: the oracle's unit
    ra = host(ac[torch.from_numpy(rows).cuda()])
    rsa = host(asc[torch.from_numpy(rows).cuda()])
    a64 = oracle.block_values_f64(ra, rsa, len(rows), K, 0)
    b64 = oracle.block_values_f64(host(bc), host(bsc), N_, K, 0)
    ref = a64 @ b64.T
    got = host(c[torch.from_numpy(rows).cuda()]).astype(np.float64)
    e = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    bound = (K * 2.0 ** -24 / (1 - K * 2.0 ** -24) + 3 * 2.0 ** -24) * (np.abs(a64) @ np.abs(b64).T)
    say("  rel-fro %.3g" % e)
    assert e <= 1e-3
    assert np.all(np.abs(got - ref) <= bound + 1e-37)
    del ac, asc, c
    torch.cuda.empty_cache()


def test_quantize_input_beyond_4gib():
    # 65600 x 32768 bf16 (4.3 GB, 2^31 + 2M elements), RHT + 1x16: input offsets pass
    # 2^32 bytes.  |x| <= 1 everywhere except one planted 100, whose transformed group holds
    # the tensor amax, so the oracle run on that row plus sampled rows (1x16 blocks: a row's
    # codes depend only on the tensor scale) reproduces the GPU's rows exactly.
    say("quantize a 4.3 GB input (65600 x 32768, RHT, 1x16)")
    rows, cols = 65600, 32768
    g = torch.Generator(device="cuda").manual_seed(3)
    xd = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, rows, 8192):   # in slabs, to bound the fp32 temporary
        r1 = min(rows, r0 + 8192)
        xd[r0:r1] = (torch.randn((r1 - r0, cols), device="cuda", generator=g) * 0.2).clamp_(-1, 1).to(torch.bfloat16)
    xd[40000, 12345] = 100.0
    q = N.quantize(xd, rht=True, rht_seed=W.RHT_SEED)
    torch.cuda.synchronize()
    sample = np.array([40000, 0, 1, 16383, 32767, 49151, 65519, 65534, 65535, 65536, 65537,
                       65550, 65570, 65590, rows - 2, rows - 1])   # 16 rows: the oracle's unit
    idx = torch.from_numpy(sample).cuda()
    xs = host(xd[idx].contiguous().view(torch.int16)).view(np.uint16)
    ref = oracle_quant(xs, rht=True, rht_seed=W.RHT_SEED)
    assert int(host(q.status)[0]) == 0
    assert host(q.global_dec)[0].view(np.uint32) == np.float32(ref[2]).view(np.uint32)
    assert np.array_equal(host(q.codes[idx]), ref[0])
    assert np.array_equal(host(q.scales[idx]), ref[1])
    del xd, q
    torch.cuda.empty_cache()


def test_quantize_16x16_with_transpose_beyond_4gib():
    # the weight path on a 4.3 GB input: 16x16 blocks with W^T from the same read.  The
    # sampled tile rows (16 rows each, one holding the planted maximum) are quantized by the
    # oracle alone; W and W^T must match it on those rows and on the matching columns of W^T.
    say("quantize a 4.3 GB input with 16x16 blocks and W^T (65600 x 32768)")
    rows, cols = 65600, 32768
    g = torch.Generator(device="cuda").manual_seed(4)
    xd = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, rows, 8192):
        r1 = min(rows, r0 + 8192)
        xd[r0:r1] = (torch.randn((r1 - r0, cols), device="cuda", generator=g) * 0.2).clamp_(-1, 1).to(torch.bfloat16)
    xd[40005, 777] = 100.0
    q = N.quantize(xd, blocking="16x16", with_transpose=True)
    torch.cuda.synchronize()
    tile_rows = np.array([2500, 0, 2047, 4095, 4096, 4099])     # 2500 * 16 = 40000 holds the max
    sample = (tile_rows[:, None] * 16 + np.arange(16)[None, :]).reshape(-1)
    idx = torch.from_numpy(sample).cuda()
    xs = host(xd[idx].contiguous().view(torch.int16)).view(np.uint16)
    ref = oracle_quant(xs, blocking="16x16")
    assert host(q.global_dec)[0].view(np.uint32) == np.float32(ref[2]).view(np.uint32)
    assert np.array_equal(host(q.codes[idx]), ref[0])
    tidx = torch.from_numpy(tile_rows).cuda()
    assert np.array_equal(host(q.scales[tidx]), ref[1])
    # W^T: columns tr*16 .. tr*16+15 of W's sampled tile rows are bytes tr*8 .. tr*8+7
    full = np.empty((len(sample), cols), np.uint8)
    full[:, 0::2], full[:, 1::2] = ref[0] & 0xF, ref[0] >> 4
    ft = np.ascontiguousarray(full.T)                            # cols x sampled rows
    want = (ft[:, 0::2] | (ft[:, 1::2] << 4)).astype(np.uint8)   # cols x 8 * len(tile_rows)
    bidx = torch.from_numpy((tile_rows[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)).cuda()
    assert np.array_equal(host(q.codes_t[:, bidx]), want)
    assert np.array_equal(host(q.scales_t[:, tidx]), np.ascontiguousarray(ref[1].T))
    del xd, q
    torch.cuda.empty_cache()


def test_quantize_sr_beyond_4gib():
    # stochastic rounding (two-pass) on a 4.3 GB input with the transform: the draws are
    # indexed by the element's global position.  Every sampled 16-row block holds a planted
    # 100 in an otherwise zero group (the tensor amax after the transform), so the oracle run
    # on that block alone, with the block's Philox index base, sees the same tensor scale
    # and the same draws.
    say("quantize a 4.3 GB input with stochastic rounding (65600 x 32768, RHT, 1x16)")
    rows, cols = 65600, 32768
    g = torch.Generator(device="cuda").manual_seed(5)
    xd = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, rows, 8192):
        r1 = min(rows, r0 + 8192)
        xd[r0:r1] = (torch.randn((r1 - r0, cols), device="cuda", generator=g) * 0.2).clamp_(-1, 1).to(torch.bfloat16)
    blocks = [0, 32768, 65520, rows - 16]
    for b0 in blocks:   # the planted group is 100 and zeros: its transformed maximum is 25
        xd[b0 + 3, 4096:4112] = 0.0   # exactly in every block (other groups stay <= 4)
        xd[b0 + 3, 4101] = 100.0
    kw = dict(rounding="sr", sr_seed=77, rht=True, rht_seed=W.RHT_SEED)
    q = N.quantize(xd, **kw)
    torch.cuda.synchronize()
    for b0 in blocks:
        xs = host(xd[b0:b0 + 16].contiguous().view(torch.int16)).view(np.uint16)
        ref = oracle_quant(xs, sr_index_base=b0 * cols, **kw)
        assert host(q.global_dec)[0].view(np.uint32) == np.float32(ref[2]).view(np.uint32)
        assert np.array_equal(host(q.codes[b0:b0 + 16]), ref[0]), b0
        assert np.array_equal(host(q.scales[b0:b0 + 16]), ref[1]), b0
    del xd, q
    torch.cuda.empty_cache()


def test_w4_full_64_seeds_exact_and_unbiased():
    """Workload 4 at its full 8192 x 5120 size with stochastic rounding seeds 0..63: every
    seed's codes, scales and tensor scale bit-exact against the oracle, and the mean over
    the 64 seeds of the stochastic codes equal to the unrounded value in code units --
    z-test |mean z| <= 5 / sqrt(n) over every non-saturated element that has two neighbours
    ([PR] outliers-and-rounding section: a value rounds up with probability equal to its
    position between the two grid points)."""
    rows, cols = 8192, 5120
    x = W.w4()
    xd = to_dev(x)
    lut = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6],
                       dtype=torch.float64, device="cuda")
    acc = torch.zeros((rows, cols), dtype=torch.float64, device="cuda")
    scales0 = g0 = None
    for s in range(64):
        say("workload 4: 8192x5120 RHT + 1x16 SR seed %d" % s)
        kw = dict(rht=True, rht_seed=W.RHT_SEED, rounding="sr", sr_seed=s)
        q = run_quant(x, xdev=xd, **kw)
        assert_same(q, oracle_quant(x, **kw))
        c = q.codes
        codes = torch.stack([c & 15, c >> 4], dim=-1).reshape(rows, cols).long()
        acc += lut[codes]
        del codes
        if scales0 is None:
            scales0, g0 = host(q.scales), host(q.global_dec)[0]
        else:   # the block and tensor scales do not depend on the draws
            assert np.array_equal(host(q.scales), scales0) and host(q.global_dec)[0] == g0
    mean = host(acc) / 64
    del acc
    y = oracle.rht16(W.bf16_bits_to_f32(x).ravel(), W.RHT_SEED).reshape(rows, cols)
    tab = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    s_enc = np.float32(2688.0) / np.float32(np.abs(y).max())
    r = (s_enc / tab[np.repeat(scales0, 16, axis=1)]).astype(np.float32)
    a = np.abs((y * r).astype(np.float64))
    del y, r
    mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    lo_i = np.clip(np.searchsorted(mags, a, side="right") - 1, 0, 6)
    lo, hi = mags[lo_i], mags[lo_i + 1]
    p = (a - lo) / (hi - lo)
    use = (a < 6) & (p > 0) & (p < 1)
    z = (np.abs(mean) - a)[use] / np.sqrt((hi - lo)[use] ** 2 * p[use] * (1 - p[use]) / 64)
    say("SR z-test: n=%d mean(z)=%.3g var(z)=%.3g" % (z.size, z.mean(), z.var()))
    assert z.size > 30_000_000   # most of the 41.9 M elements take part
    assert abs(z.mean()) <= 5 / np.sqrt(z.size)
