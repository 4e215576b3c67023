"""GPU parity of the MXFP4 path (quantize, dequantize, native FP4 MFMA GEMM) against the
CPU oracle, through the C ABI.

Codes and scales bit-exact; dequantized values bit-exact; the GEMM within 1e-3 relative
Frobenius of the binary64 product and inside the fp32 summation bound per element.  Also
the pages' comparison of the two formats, measured on the GPU path: NVFP4's 16-element
E4M3 blocks against MXFP4's 32-element E8M0 blocks, per-block error and GEMM error.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from block_scaled_fp4_06_amd import nvfp4 as N  # noqa: E402
from block_scaled_fp4_06_amd import workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu


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


def mx_run(x_u16, xdev=None):
    q = N.mx_quantize(to_dev(x_u16) if xdev is None else xdev)
    torch.cuda.synchronize()
    return q


def assert_mx_same(q, x_u16):
    codes, scales, _ = oracle.mx_quantize(x_u16)
    gs = host(q.scales)
    if not np.array_equal(gs, scales):
        bad = np.argwhere(gs != scales)
        raise AssertionError("%d scales differ, first at %s: gpu %d oracle %d" % (
            len(bad), bad[0], gs[tuple(bad[0])], scales[tuple(bad[0])]))
    gc = host(q.codes)
    if not np.array_equal(gc, codes):
        bad = np.argwhere(gc != codes)
        raise AssertionError("%d code bytes differ, first at %s: gpu %02x oracle %02x" % (
            len(bad), bad[0], gc[tuple(bad[0])], codes[tuple(bad[0])]))
    return codes, scales


MX_SHAPES = [(1, 32), (7, 64), (33, 96), (272, 544), (1040, 2080), (3, 4128)]


@pytest.mark.parametrize("rows,cols", MX_SHAPES)
def test_mx_quantize_shapes(rows, cols):
    say("mx quantize %dx%d" % (rows, cols))
    x = W.channel_outliers(rows, cols, seed=rows * 7 + cols)
    assert_mx_same(mx_run(x), x)
    y = W.student_t(rows, cols, seed=rows + cols)
    assert_mx_same(mx_run(y), y)


def test_mx_quantize_row_stride():
    say("mx quantize with row stride 200 > cols 160")
    full = W.normal_outliers(64, 200, seed=11)
    xd = to_dev(full)[:, :160]
    q = mx_run(None, xdev=xd)
    assert_mx_same(q, np.ascontiguousarray(full[:, :160]))


def test_mx_edge_values():
    say("mx edge values: zero, -0, subnormal, huge, midpoints, non-finite blocks")
    rng = np.random.default_rng(3)
    x = W.f32_to_bf16_bits(rng.standard_normal((16, 256)).astype(np.float32))
    x[0, :32] = 0                                    # all-zero block
    x[1, :32] = 0x8000                               # all -0
    x[2, :32] = 0x0001                               # smallest subnormal bf16
    x[2, 32:64] = rng.integers(0, 0x80, 32)          # subnormal block (scale byte 0)
    x[3, :32] = 0x7F7F                               # largest finite bf16 (scale 252)
    x[3, 40] = 0xFF7F
    x[4, :32] = 0x7F80                               # +inf block
    x[4, 64] = 0xFFC0                                # a NaN in another block
    x[5, :32] = W.f32_to_bf16_bits(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0] * 4,
                                            np.float32) * 2.0 ** 10)   # E2M1 midpoints
    x[6, :32] = W.f32_to_bf16_bits(np.array([-0.25, -0.1, 6.0, 7.9] * 8, np.float32))
    x[7, :32] = W.f32_to_bf16_bits(np.full(32, 2.0 ** -126, np.float32))   # clamps at 2^-127
    x[8, :32] = W.f32_to_bf16_bits(np.full(32, 2.0 ** -125, np.float32))
    codes, scales = assert_mx_same(mx_run(x), x)
    assert scales[0, 0] == 0 and scales[4, 0] == 0xFF and scales[4, 2] == 0xFF
    assert np.all(codes[4, :16] == 0)
    assert scales[3, 0] == 252


def test_mx_quantize_w3_full():
    say("mx quantize workload 3 (8192x5120 activations with channel outliers)")
    x = W.w3()
    assert_mx_same(mx_run(x), x)


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_mx_dequantize_parity(out):
    say("mx dequantize, every scale byte, %s out" % out)
    rng = np.random.default_rng(17)
    rows, cols = 64, 1024
    codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (rows, cols // 32), dtype=np.uint8)
    scales.reshape(-1)[:256] = np.arange(256, dtype=np.uint8)
    with np.errstate(over="ignore"):   # scale bytes near 254 overflow binary32: inf, as in the kernel
        ref = oracle.mx_block_values_f64(codes, scales, rows, cols).astype(np.float32)
    q = N.MXFP4Tensor(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), rows, cols)
    if out == "f32":
        y = host(N.mx_dequantize(q, torch.float32))
        got = y.view(np.uint32)
        exp = ref.view(np.uint32)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(y), nan)
        assert np.array_equal(got[~nan], exp[~nan])
    else:
        y = host(N.mx_dequantize(q, torch.bfloat16).view(torch.int16)).view(np.uint16)
        exp = W.f32_to_bf16_bits(ref)
        nan = np.isnan(ref)
        assert np.array_equal((y & 0x7FFF) > 0x7F80, nan)
        assert np.array_equal(y[~nan], exp[~nan])
    # strided output
    yd = torch.zeros((rows, cols + 64), dtype=torch.float32, device="cuda")
    N.mx_dequantize(q, out=yd[:, :cols])
    ys = host(yd)
    assert np.all(ys[:, cols:] == 0)
    nan = np.isnan(ref)
    assert np.array_equal(ys[:, :cols][~nan].view(np.uint32), ref[~nan].view(np.uint32))


def mx_gemm_check(qa, qb, ref_a, ref_b, M, N_, K, rows=None):
    c32 = N.mx_gemm(qa, qb, torch.float32)
    cb = N.mx_gemm(qa, qb, torch.bfloat16)
    torch.cuda.synchronize()
    sl = rows if rows is not None else slice(None)
    a_t = (ref_a[0], ref_a[1], M, K)
    b_t = (ref_b[0], ref_b[1], N_, K)
    cref = oracle.mx_gemm_reference(a_t, b_t, row_slice=sl)
    g32 = host(c32)[sl].astype(np.float64)
    gb = W.bf16_bits_to_f32(host(cb.view(torch.int16)).view(np.uint16)[sl]).astype(np.float64)
    fro = np.linalg.norm(cref)
    e32 = np.linalg.norm(g32 - cref) / max(fro, 1e-300)
    cref_bf16 = W.bf16_bits_to_f32(W.f32_to_bf16_bits(cref.astype(np.float32))).astype(np.float64)
    eb = np.linalg.norm(gb - cref_bf16) / max(np.linalg.norm(cref_bf16), 1e-300)
    say("mx gemm %dx%dx%d: rel-fro fp32 %.3g, bf16 vs bf16(ref) %.3g" % (M, N_, K, e32, eb))
    assert e32 <= 1e-3
    assert eb <= 1e-3
    # per element: |fl(sum) - sum| <= gamma_K * sum |a||b|, plus one rounding to fp32
    qa64 = oracle.mx_block_values_f64(*a_t)[sl]
    qb64 = oracle.mx_block_values_f64(*b_t)
    absprod = np.abs(qa64) @ np.abs(qb64).T
    u = 2.0 ** -24
    bound = (K * u / (1 - K * u) + u) * absprod + 1e-37
    assert np.all(np.abs(g32 - cref) <= bound)
    return e32


MX_GEMM_SHAPES = [(32, 32, 32), (48, 80, 96), (256, 256, 256), (300, 260, 288),
                  (64, 512, 800), (520, 264, 512), (1040, 784, 2304), (16, 2000, 1024)]


@pytest.mark.parametrize("M,N_,K", MX_GEMM_SHAPES)
def test_mx_gemm_small(M, N_, K):
    say("mx gemm %dx%dx%d" % (M, N_, K))
    a = W.channel_outliers(M, K, seed=M + K)
    b = W.normal_scaled(N_, K, seed=N_ + K, std=0.02)
    qa, qb = mx_run(a), mx_run(b)
    ra, rb = assert_mx_same(qa, a), assert_mx_same(qb, b)
    mx_gemm_check(qa, qb, ra, rb, M, N_, K)


def test_mx_gemm_k_zero_and_empty():
    say("mx gemm K = 0 writes zeros; M = 0 is a no-op")
    qa = N.MXFP4Tensor(torch.empty((40, 0), dtype=torch.uint8, device="cuda"),
                       torch.empty((40, 0), dtype=torch.uint8, device="cuda"), 40, 0)
    qb = N.MXFP4Tensor(torch.empty((24, 0), dtype=torch.uint8, device="cuda"),
                       torch.empty((24, 0), dtype=torch.uint8, device="cuda"), 24, 0)
    c = torch.full((40, 24), 7.0, device="cuda")
    N.mx_gemm(qa, qb, out=c)
    torch.cuda.synchronize()
    assert torch.all(c == 0)
    e = N.mx_gemm(N.MXFP4Tensor(qa.codes[:0], qa.scales[:0], 0, 0), qb, torch.float32)
    assert e.shape == (0, 24)


def test_mx_gemm_nan_scale_poisons_its_row():
    say("mx gemm with a non-finite block in A")
    M, N_, K = 64, 64, 256
    a = W.normal_scaled(M, K, seed=1, std=1.0)
    a[5, 40] = 0x7F80
    b = W.normal_scaled(N_, K, seed=2, std=1.0)
    qa, qb = mx_run(a), mx_run(b)
    ra, rb = assert_mx_same(qa, a), assert_mx_same(qb, b)
    c = host(N.mx_gemm(qa, qb, torch.float32))
    cref = oracle.mx_gemm_reference((ra[0], ra[1], M, K), (rb[0], rb[1], N_, K))
    assert np.array_equal(np.isnan(c), np.isnan(cref))
    ok = ~np.isnan(cref)
    assert np.allclose(c[ok], cref[ok], rtol=1e-5, atol=1e-5)


def test_mx_gemm_w5_full_sampled():
    say("mx workload 5: 8192x5120 . (20480x5120)^T GEMM, sampled rows")
    a = W.w3()
    wt = np.ascontiguousarray(W.w5_weight().T)   # N x K
    qa, qb = mx_run(a), mx_run(wt)
    ra, rb = assert_mx_same(qa, a), assert_mx_same(qb, wt)
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(8192, 48, replace=False))
    mx_gemm_check(qa, qb, ra, rb, 8192, 20480, 5120, rows=rows)


def test_mx_gemm_operand_beyond_2gib():
    # A of 524800 x 8192 MXFP4 codes (2.15 GB): rows past the 2^31-byte mark are read
    say("mx gemm with a 2.15 GB operand")
    M, N_, K = 524800, 256, 8192
    g = torch.Generator(device="cuda").manual_seed(2)
    ac = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    asc = torch.randint(120, 134, (M, K // 32), dtype=torch.uint8, device="cuda", generator=g)
    bc = torch.randint(0, 256, (N_, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    bsc = torch.randint(120, 134, (N_, K // 32), dtype=torch.uint8, device="cuda", generator=g)
    c = N.mx_gemm(N.MXFP4Tensor(ac, asc, M, K), N.MXFP4Tensor(bc, bsc, N_, K), torch.float32)
    torch.cuda.synchronize()
    rows = np.array([0, 262144, 524287, 524288, 524289, 524544, M - 1])
    idx = torch.from_numpy(rows).cuda()
    a64 = oracle.mx_block_values_f64(host(ac[idx]), host(asc[idx]), len(rows), K)
    b64 = oracle.mx_block_values_f64(host(bc), host(bsc), N_, K)
    ref = a64 @ b64.T
    got = host(c[torch.from_numpy(rows).cuda()]).astype(np.float64)
    e = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    say("  rel-fro %.3g" % e)
    assert e <= 1e-3
    bound = (K * 2.0 ** -24 / (1 - K * 2.0 ** -24) + 2.0 ** -24) * (np.abs(a64) @ np.abs(b64).T)
    assert np.all(np.abs(got - ref) <= bound + 1e-37)
    del ac, asc, c
    torch.cuda.empty_cache()


def test_format_comparison_on_gpu():
    # The pages' claim (16-element E4M3 blocks quantize more accurately than 32-element
    # E8M0 blocks), measured on the GPU path: per-block max error and relative Frobenius
    # error of the dequantized workload-1 and workload-3 tensors, and the error of the
    # workload-5 product against the exact product of the bf16 inputs.
    for name, x in (("w1", W.w1()), ("w3", W.w3())):
        rows, cols = x.shape
        xd = to_dev(x)
        xf = xd.double()
        nv = N.dequantize(N.quantize(xd), torch.float32).double()
        mx = N.mx_dequantize(N.mx_quantize(xd), torch.float32).double()
        e_nv, e_mx = (nv - xf).abs(), (mx - xf).abs()
        fro_nv = float(e_nv.norm() / xf.norm())
        fro_mx = float(e_mx.norm() / xf.norm())
        # per 32-element block: max error of each format
        b_nv = e_nv.view(rows, cols // 32, 32).amax(-1)
        b_mx = e_mx.view(rows, cols // 32, 32).amax(-1)
        better = float((b_nv < b_mx).double().mean())
        say("formats %s: rel-fro nvfp4 %.4f mxfp4 %.4f | nvfp4 block max err lower in %.1f%% "
            "of 32-blocks" % (name, fro_nv, fro_mx, 100 * better))
        assert fro_nv < fro_mx
        assert better > 0.5


def test_format_comparison_gemm_error():
    # The same comparison at the product: the workload-5 GEMM (activations 8192 x 5120 with
    # channel outliers, the 5120 x 20480 weight) in NVFP4 (1x16 activations, 16x16 weight)
    # and in MXFP4, each against the exact product of the bf16 inputs on sampled rows.
    say("formats at the product: workload-5 GEMM error, NVFP4 vs MXFP4")
    x = W.w3()
    w = W.w5_weight()
    wt = np.ascontiguousarray(w.T)
    xd, wd, wtd = to_dev(x), to_dev(w), to_dev(wt)
    rows = np.sort(np.random.default_rng(9).choice(8192, 64, replace=False))
    idx = torch.from_numpy(rows).cuda()
    exact = W.bf16_bits_to_f32(x[rows]).astype(np.float64) @ W.bf16_bits_to_f32(w).astype(np.float64)
    qx = N.quantize(xd)
    qw = N.quantize(wd, blocking="16x16", with_transpose=True)
    c_nv = host(N.gemm(qx, qw.transposed(), torch.float32)[idx]).astype(np.float64)
    c_mx = host(N.mx_gemm(N.mx_quantize(xd), N.mx_quantize(wtd), torch.float32)[idx]).astype(np.float64)
    e_nv = np.linalg.norm(c_nv - exact) / np.linalg.norm(exact)
    e_mx = np.linalg.norm(c_mx - exact) / np.linalg.norm(exact)
    say("  GEMM rel-fro error vs the exact bf16 product: nvfp4 %.4f, mxfp4 %.4f" % (e_nv, e_mx))
    assert e_nv < e_mx


def test_mx_gemm_edge_blocks_and_strided_output():
    # K = 288 (a partial last step of 32 elements), a non-finite block inside that partial
    # step, all-zero blocks, and C written into a wider row-strided buffer
    say("mx gemm edge blocks: partial last K step with a NaN block, zero blocks, strided C")
    M, N_, K = 96, 80, 288
    a = W.normal_scaled(M, K, seed=21, std=1.0)
    b = W.normal_scaled(N_, K, seed=22, std=0.1)
    a[7, 270] = 0x7FC0          # NaN in the last 32-element block of row 7
    a[9, :] = 0                 # a zero row (every scale byte 0)
    b[3, 32:64] = 0x8000        # a block of -0 in B
    qa, qb = mx_run(a), mx_run(b)
    ra, rb = assert_mx_same(qa, a), assert_mx_same(qb, b)
    full = torch.full((M, N_ + 24), 5.0, dtype=torch.float32, device="cuda")
    N.mx_gemm(qa, qb, out=full[:, :N_])
    torch.cuda.synchronize()
    c = host(full)
    assert np.all(c[:, N_:] == 5.0)
    cref = oracle.mx_gemm_reference((ra[0], ra[1], M, K), (rb[0], rb[1], N_, K))
    got = c[:, :N_]
    assert np.array_equal(np.isnan(got), np.isnan(cref))
    assert np.all(np.isnan(got[7]))
    assert np.all(got[9] == 0)
    ok = ~np.isnan(cref)
    qa64 = oracle.mx_block_values_f64(ra[0], ra[1], M, K)
    qb64 = oracle.mx_block_values_f64(rb[0], rb[1], N_, K)
    bound = (K * 2.0 ** -24 / (1 - K * 2.0 ** -24) + 2.0 ** -24) * (np.nan_to_num(np.abs(qa64)) @ np.abs(qb64).T) + 1e-37
    assert np.all(np.abs(got[ok] - cref[ok]) <= bound[ok])
