"""Seeded synthetic inputs for the NVFP4 quantize / GEMM workloads.

This module only draws random numbers and rounds them once to bfloat16; it holds none
of the quantization arithmetic, so the CPU oracle and the GPU library can both be fed
from it without sharing any code.  The pages measure no public dataset: every input is
synthetic, with the distributions the five workloads name:

  W1  256 x 256,    N(0, 1), 0.1 % of the entries (66 seeded positions) times 100
  W2  4096 x 4096,  N(0, 0.02^2)                                   (a weight matrix)
  W3  8192 x 5120,  N(0, 1), 8 seeded channels (columns) times 50  (activations)
  W4  8192 x 5120,  Student-t with 3 degrees of freedom, times 1e-3 (gradients)
  W5  activations as W3 times a 5120 x 20480 weight drawn as W2 (seed 5)

Values are drawn in float32 with numpy's PCG64 ``default_rng(seed)``, scaled in float32,
then rounded once to bfloat16 (round to nearest, ties to even).  bfloat16 tensors are
returned as uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

RHT_SEED = 0x5248
SEEDS = {"w1": 1, "w2": 2, "w3": 3, "w4": 4, "w5_weight": 5}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_outliers(rows: int, cols: int, seed: int, frac: float = 0.001,
                    factor: float = 100.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    k = int(round(frac * rows * cols))
    pos = rng.choice(rows * cols, k, replace=False)
    x.reshape(-1)[pos] *= np.float32(factor)
    return f32_to_bf16_bits(x)


def normal_scaled(rows: int, cols: int, seed: int, std: float) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    x *= np.float32(std)
    return f32_to_bf16_bits(x)


def channel_outliers(rows: int, cols: int, seed: int, nchan: int = 8,
                     factor: float = 50.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    ch = rng.choice(cols, nchan, replace=False)
    x[:, ch] *= np.float32(factor)
    return f32_to_bf16_bits(x)


def student_t(rows: int, cols: int, seed: int, nu: float = 3.0,
              scale: float = 1e-3) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_t(nu, (rows, cols)).astype(np.float32)
    x *= np.float32(scale)
    return f32_to_bf16_bits(x)


def w1(rows: int = 256, cols: int = 256) -> np.ndarray:
    return normal_outliers(rows, cols, SEEDS["w1"])


def w2(rows: int = 4096, cols: int = 4096) -> np.ndarray:
    return normal_scaled(rows, cols, SEEDS["w2"], 0.02)


def w3(rows: int = 8192, cols: int = 5120) -> np.ndarray:
    return channel_outliers(rows, cols, SEEDS["w3"])


def w4(rows: int = 8192, cols: int = 5120) -> np.ndarray:
    return student_t(rows, cols, SEEDS["w4"])


def w5_weight(k: int = 5120, n: int = 20480) -> np.ndarray:
    """The K x N weight of the linear-layer workload (as W2, seed 5)."""
    return normal_scaled(k, n, SEEDS["w5_weight"], 0.02)


# Quantization parameters of each workload (blocking, rounding, RHT).
PARAMS = {
    "w1": dict(blocking="1x16", rounding="rne", rht=False),
    "w2": dict(blocking="16x16", rounding="rne", rht=False),
    "w3": dict(blocking="1x16", rounding="rne", rht=True, rht_seed=RHT_SEED),
    "w4": dict(blocking="1x16", rounding="sr", rht=True, rht_seed=RHT_SEED),
    "w5_act": dict(blocking="1x16", rounding="rne", rht=True, rht_seed=RHT_SEED),
    "w5_weight": dict(blocking="16x16", rounding="rne", rht=False),
}
