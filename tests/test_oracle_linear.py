"""Pins of the oracle's linear-layer composition (Fprop, Dgrad, Wgrad on quantized
operands) against facts that do not come from the oracle itself.

* Inputs whose every 16-element row group holds a value of magnitude 6 * 2^e and whose
  other values lie on the E2M1 grid times 2^e quantize losslessly under the recipe (the
  tensor scale makes every block scale exactly 448), and stochastic rounding of an exactly
  representable value cannot move it.  So Fprop and Dgrad must equal the exact binary64
  products X W and dY W^T, element for element, up to the rounding of the FP32 tensor
  scales (a factor within 2^-24 of 1 per operand): a transposed operand, the wrong weight
  layout or a dropped tensor scale fails this.
* Wgrad quantizes the transformed X^T and dY^T; the transform (same seed on both) keeps
  the product, so dW stays within the FP4 error of X^T dY, while transforms with different
  seeds (a planted mistake) destroy it.
"""
import numpy as np

import oracle
from block_scaled_fp4_06_amd import workloads as W

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def representable(rows, cols, e, seed):
    rng = np.random.default_rng(seed)
    v = rng.choice(E2M1, size=(rows, cols)) * rng.choice([-1.0, 1.0], size=(rows, cols))
    # one element of magnitude 6 in every 16-element row group
    pos = rng.integers(0, 16, size=(rows, cols // 16))
    for g in range(cols // 16):
        v[np.arange(rows), 16 * g + pos[:, g]] = 6.0 * rng.choice([-1.0, 1.0], size=rows)
    v *= 2.0 ** e
    return W.f32_to_bf16_bits(v.astype(np.float32)), v


def test_fprop_dgrad_exact_on_representable_inputs():
    M, K, N = 48, 64, 80
    x, xf = representable(M, K, -3, 1)
    w, wf = representable(K, N, -6, 2)
    dy, dyf = representable(M, N, -12, 3)
    y, dx, dw = oracle.linear_reference(x, w, dy, rht_seed=0x5248, sr_seed=9)
    # every block scale is 448 and the codes are exact; the only rounding is the FP32
    # tensor scale amax / 2688 = 2^e / 448, so each operand carries a factor
    # c = 448 g / 2^e within 2^-24 of 1
    gx = float(oracle.quantize(x)[2])
    gw = float(oracle.quantize(w, blocking=oracle.BLOCK_16x16)[2])
    gd = float(oracle.quantize(dy, rounding=oracle.ROUND_SR, sr_seed=9)[2])
    cx, cw, cd = 448 * gx / 2.0 ** -3, 448 * gw / 2.0 ** -6, 448 * gd / 2.0 ** -12
    for c in (cx, cw, cd):
        assert abs(c - 1) <= 2.0 ** -24
    assert np.allclose(y, (xf @ wf) * (cx * cw), rtol=1e-14, atol=0)
    assert np.allclose(dx, (dyf @ wf.T) * (cd * cw), rtol=1e-14, atol=0)
    exact = xf.T @ dyf
    assert np.linalg.norm(dw - exact) / np.linalg.norm(exact) < 0.25


def test_wgrad_keeps_the_product_only_with_matching_transforms():
    M, K, N = 256, 48, 32
    x = W.channel_outliers(M, K, seed=4)
    dy = W.normal_scaled(M, N, seed=5, std=1e-3)
    w = W.normal_scaled(K, N, seed=6, std=0.05)
    f = lambda a: W.bf16_bits_to_f32(a).astype(np.float64)
    exact = f(x).T @ f(dy)
    _, _, dw = oracle.linear_reference(x, w, dy, rht_seed=0x5248, sr_seed=1)
    good = np.linalg.norm(dw - exact) / np.linalg.norm(exact)
    # planted mistake: the two Wgrad operands transformed with different sign vectors
    qxt = oracle.quantize(np.ascontiguousarray(x.T), rht=True, rht_seed=0x5248)
    qdyt = oracle.quantize(np.ascontiguousarray(dy.T), rounding=oracle.ROUND_SR, rht=True,
                           rht_seed=0x1234, sr_seed=2)
    bad_dw = oracle.gemm_reference((*qxt[:3], K, M, 0), (*qdyt[:3], N, M, 0))
    bad = np.linalg.norm(bad_dw - exact) / np.linalg.norm(exact)
    assert good < 0.25
    assert bad > 0.6


def test_operands_shapes_and_shared_weight_quantization():
    M, K, N = 32, 48, 64
    x = W.normal_scaled(M, K, seed=7, std=1.0)
    w = W.normal_scaled(K, N, seed=8, std=0.05)
    dy = W.normal_scaled(M, N, seed=9, std=1e-3)
    qx, qwt, qw, qdy, qxt, qdyt = oracle.linear_operands(x, w, dy, 0x5248, 3)
    assert qx[0].shape == (M, K // 2) and qwt[0].shape == (N, K // 2)
    assert qw[0].shape == (K, N // 2) and qdy[0].shape == (M, N // 2)
    assert qxt[0].shape == (K, M // 2) and qdyt[0].shape == (N, M // 2)
    # with 16x16 blocks the quantized W^T is the transposed quantized W (same tensor
    # scale, same block scales transposed, same codes transposed)
    assert qwt[2] == qw[2]
    assert np.array_equal(qwt[1], qw[1].T)
    full = np.empty((K, N), np.uint8)
    full[:, 0::2], full[:, 1::2] = qw[0] & 0xF, qw[0] >> 4
    ft = full.T
    assert np.array_equal(qwt[0], (ft[:, 0::2] | (ft[:, 1::2] << 4)).astype(np.uint8))
