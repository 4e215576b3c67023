"""GPU parity of the NVFP4 linear layer (Fprop, Dgrad, Wgrad) and of the bf16 transpose
against the CPU oracle, through the C ABI.

Every quantized operand of the three products (X, W with its transpose, dY, X^T, dY^T)
must match the oracle bit for bit; each product within 1e-3 relative Frobenius of the
oracle's binary64 product and inside the fp32 summation bound per element.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from block_scaled_fp4_06_amd import linear as L  # noqa: E402
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


def to_dev(x_u16):
    return torch.from_numpy(np.ascontiguousarray(x_u16).view(np.int16)).view(torch.bfloat16).cuda()


def host(t):
    return t.cpu().numpy()


def bits(t):
    return host(t.contiguous().view(torch.int16)).view(np.uint16)


@pytest.mark.parametrize("rows,cols", [(8, 8), (16, 32), (72, 136), (1000, 520), (64, 4104)])
def test_transpose_parity(rows, cols):
    say("transpose %dx%d" % (rows, cols))
    x = W.normal_outliers(rows, cols, seed=rows + cols)
    y = N.transpose(to_dev(x))
    torch.cuda.synchronize()
    assert y.shape == (cols, rows)
    assert np.array_equal(bits(y), np.ascontiguousarray(x.T))


def test_transpose_strided():
    say("transpose with row strides on both sides")
    full = W.normal_outliers(40, 200, seed=3)
    xd = to_dev(full)[:, :168]
    out = torch.zeros((168, 56), dtype=torch.bfloat16, device="cuda")
    N.transpose(xd, out=out[:, :40])
    torch.cuda.synchronize()
    o = bits(out)
    assert np.array_equal(o[:, :40], np.ascontiguousarray(full[:, :168].T))
    assert np.all(o[:, 40:] == 0)


def same_q(q, ref, what):
    codes, scales, g, _ = ref
    assert np.float32(host(q.global_dec)[0]).view(np.uint32) == np.float32(g).view(np.uint32), what
    assert np.array_equal(host(q.scales), scales), what
    assert np.array_equal(host(q.codes), codes), what


def check_product(got, ref_c, qa64, qb64, K, rows, name):
    g = host(got)[rows].astype(np.float64)
    r = ref_c
    e = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
    absprod = np.abs(qa64) @ np.abs(qb64).T
    u = 2.0 ** -24
    bound = (K * u / (1 - K * u) + 3 * u) * absprod + 1e-37
    say("  %s: rel-fro %.3g" % (name, e))
    assert e <= 1e-3, name
    assert np.all(np.abs(g - r) <= bound), name


def run_layer(M, K, N_, seed, rows=None):
    x = W.channel_outliers(M, K, seed=seed)
    w = W.normal_scaled(K, N_, seed=seed + 1, std=0.02)
    dy = W.student_t(M, N_, seed=seed + 2, scale=1e-3)
    xd, wd, dyd = to_dev(x), to_dev(w), to_dev(dy)
    rs, ss = L.DEFAULT_RHT_SEED, 11
    y, ctx = L.linear_forward(xd, wd, rht_seed=rs, sr_seed=ss, out_dtype=torch.float32)
    dx, dw = L.linear_backward(dyd, ctx, dx_dtype=torch.float32, dw_dtype=torch.float32)
    torch.cuda.synchronize()
    ops = oracle.linear_operands(x, w, dy, rs, ss)
    qx, qwt, qw, qdy, qxt, qdyt = ops
    # the operands the GPU path quantized, recomputed from its own calls' inputs
    same_q(N.quantize(xd), qx, "X")
    same_q(ctx.qw, qw, "W")
    same_q(ctx.qw.transposed(), qwt, "W^T")
    same_q(N.quantize(dyd, rounding="sr", sr_seed=ss), qdy, "dY")
    same_q(N.quantize(N.transpose(xd), rht=True, rht_seed=rs), qxt, "X^T")
    same_q(N.quantize(N.transpose(dyd), rounding="sr", rht=True, rht_seed=rs, sr_seed=ss + 1),
           qdyt, "dY^T")
    sl = rows if rows is not None else slice(None)
    bv = oracle.block_values_f64
    # Fprop
    a64 = bv(*qx[:2], M, K, 0)[sl] * float(qx[2])
    b64 = bv(*qwt[:2], N_, K, 1) * float(qwt[2])
    check_product(y, a64 @ b64.T, a64, b64, K, sl, "Y = X W")
    # Dgrad
    a64 = bv(*qdy[:2], M, N_, 0)[sl] * float(qdy[2])
    b64 = bv(*qw[:2], K, N_, 1) * float(qw[2])
    check_product(dx, a64 @ b64.T, a64, b64, N_, sl, "dX = dY W^T")
    # Wgrad (rows of dW are K)
    slk = rows if rows is None else np.sort(np.random.default_rng(1).choice(K, len(rows), replace=False))
    slk = slk if slk is not None else slice(None)
    a64 = bv(*qxt[:2], K, M, 0)[slk] * float(qxt[2])
    b64 = bv(*qdyt[:2], N_, M, 0) * float(qdyt[2])
    check_product(dw, a64 @ b64.T, a64, b64, M, slk, "dW = X^T dY")
    return x, w, dy, y, dx, dw


@pytest.mark.parametrize("M,K,N_", [(64, 96, 80), (272, 528, 144), (1040, 512, 784)])
def test_linear_layer_parity(M, K, N_):
    say("linear layer M=%d K=%d N=%d" % (M, K, N_))
    run_layer(M, K, N_, seed=M + K + N_)


def test_linear_layer_workload5_sampled():
    say("linear layer at workload-5 size: X 8192x5120, W 5120x20480, dY 8192x20480")
    rows = np.sort(np.random.default_rng(7).choice(8192, 32, replace=False))
    run_layer(8192, 5120, 20480, seed=5, rows=rows)


def test_autograd_function_matches_the_calls():
    say("autograd function: backward gives the library's dX and dW")
    M, K, N_ = 128, 256, 192
    x = to_dev(W.normal_scaled(M, K, seed=1, std=1.0)).requires_grad_(True)
    w = to_dev(W.normal_scaled(K, N_, seed=2, std=0.05)).requires_grad_(True)
    dy = to_dev(W.normal_scaled(M, N_, seed=3, std=1e-3))
    Fn = L.autograd_linear()
    y = Fn.apply(x, w, L.DEFAULT_RHT_SEED, 5)
    y.backward(dy)
    y2, ctx = L.linear_forward(x.detach(), w.detach(), sr_seed=5)
    dx2, dw2 = L.linear_backward(dy, ctx, dw_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), y2)
    assert torch.equal(x.grad, dx2)
    assert torch.equal(w.grad, dw2)
    # and the layer approximates the exact products of its bf16 inputs
    xf, wf, df = x.detach().double(), w.detach().double(), dy.double()
    for got, exact in ((y2, xf @ wf), (dx2, df @ wf.T), (dw2, xf.T @ df)):
        e = float((got.double() - exact).norm() / exact.norm())
        assert e < 0.25


def test_dgrad_stochastic_rounding_is_unbiased():
    # Why the recipe rounds gradients stochastically: averaged over seeds, dX = q(dY) W^T
    # converges to dY W_q^T (the error of one draw shrinks ~1/sqrt(n)), while nearest-even
    # rounding of dY leaves a fixed bias that no averaging removes.
    say("Dgrad with SR: the mean over 32 seeds approaches dY W_q^T; RNE does not")
    M, K, N_ = 256, 512, 384
    x = to_dev(W.normal_scaled(M, K, seed=31, std=1.0))
    w = to_dev(W.normal_scaled(K, N_, seed=32, std=0.05))
    dy = to_dev(W.student_t(M, N_, seed=33))
    _, ctx = L.linear_forward(x, w)
    qw = ctx.qw
    wq = torch.from_numpy(oracle.block_values_f64(host(qw.codes), host(qw.scales), K, N_, 1)
                          * float(host(qw.global_dec)[0])).cuda()
    target = dy.double() @ wq.T                     # the unquantized-gradient product
    nrm = float(target.norm())
    acc = torch.zeros_like(target)
    single = None
    for s in range(32):
        qdy = N.quantize(dy, rounding="sr", sr_seed=s)
        dx = N.gemm(qdy, qw, torch.float32).double()
        acc += dx
        if single is None:
            single = float((dx - target).norm()) / nrm
    mean_err = float((acc / 32 - target).norm()) / nrm
    rne = N.gemm(N.quantize(dy), qw, torch.float32).double()
    rne_err = float((rne - target).norm()) / nrm
    say("  rel-fro vs dY W_q^T: one SR draw %.4f, mean of 32 SR draws %.4f, nearest-even %.4f"
        % (single, mean_err, rne_err))
    assert mean_err < single / 3
    assert mean_err < rne_err / 2
