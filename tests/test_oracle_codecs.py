"""Pins for the oracle's E2M1 / E4M3 / bfloat16 codecs (CPU only).

Each test checks the oracle against something other than itself: values the pages
print (tests/golden/pages_facts.json), torch's float8_e4m3fn and bfloat16 casts
(library routines), and exhaustive or exact-rational brute force.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
FACTS = json.load(open(os.path.join(HERE, "golden", "pages_facts.json")))


def f32_range(lo: float, hi: float) -> np.ndarray:
    """Every binary32 value in [lo, hi] (both >= 0), ascending."""
    a = np.array([lo], np.float32).view(np.uint32)[0]
    b = np.array([hi], np.float32).view(np.uint32)[0]
    return np.arange(a, b + 1, dtype=np.uint32).view(np.float32)


# ------------------------------------------------------------------ E2M1
def test_e2m1_value_set(orc):
    vals = orc.e2m1_decode(range(16))
    mags = FACTS["e2m1_magnitudes"]["value"]
    assert list(vals[:8]) == mags
    assert list(vals[8:]) == [-m for m in mags]
    assert np.signbit(vals[8])  # code 8 is -0
    assert len(set(map(float, vals))) == 15  # 16 codes, +0 and -0 compare equal


def test_block_scale_example_600(orc):
    """PR: the 4-bit value 6 with a block scale of 100 stands for 600.  With the
    two-level scale, 100 = sbd * s_dec with sbd = 5 (E4M3 code 0x4A) and s_dec = 20."""
    f = FACTS["block_scale_example"]
    code6 = [c for c in range(8) if orc.e2m1_decode([c])[0] == f["element"]][0]
    assert orc.e4m3_decode([0x4A])[0] == 5.0
    codes = np.full((16, 8), code6 | (code6 << 4), np.uint8)
    scales = np.full((16, 1), 0x4A, np.uint8)
    y = orc.dequantize(codes, scales, 20.0, 16, 16, orc.BLOCK_1x16)
    assert 5.0 * 20.0 == f["scale"]
    assert np.all(y == f["value"])


def _rn_reference_by_thresholds(a: np.ndarray) -> np.ndarray:
    """Nearest E2M1 magnitude code written as decision intervals.  The boundaries are
    the midpoints between neighbours; a value exactly on a midpoint goes to the
    neighbour whose code is even (mantissa bit 0):
      [0, .25] -> 0   (.25, .75) -> 1   [.75, 1.25] -> 2   (1.25, 1.75) -> 3
      [1.75, 2.5] -> 4   (2.5, 3.5) -> 5   [3.5, 5] -> 6   (5, inf) -> 7"""
    code = np.zeros(a.shape, np.uint8)
    code += (a > 0.25)
    code += (a >= 0.75)
    code += (a > 1.25)
    code += (a >= 1.75)
    code += (a > 2.5)
    code += (a >= 3.5)
    code += (a > 5.0)
    return code


def test_e2m1_rn_exhaustive(orc):
    """Every binary32 in [2^-4, 8] (58 M values) plus a sample below 2^-4 and above 8."""
    a = f32_range(2.0 ** -4, 8.0)
    for i in range(0, a.size, 1 << 23):
        chunk = a[i:i + (1 << 23)]
        assert np.array_equal(orc.e2m1_encode_rn(chunk), _rn_reference_by_thresholds(chunk))
    rng = np.random.default_rng(11)
    small = (rng.random(1 << 20, dtype=np.float32) * np.float32(2.0 ** -4))
    small = np.concatenate([small, np.array([0.0, 1e-45, 1e-38], np.float32)])
    assert np.all(orc.e2m1_encode_rn(small) == 0)
    big = np.array([8.0, 100.0, 3.0e38, np.inf], np.float32)
    assert np.all(orc.e2m1_encode_rn(big) == 7)


def test_e2m1_rn_sign_and_exact_rational(orc):
    """Negative inputs set the sign bit only; nearest-value check in exact rationals for
    midpoints and their binary32 neighbours."""
    mags = [Fraction(m).limit_denominator() for m in FACTS["e2m1_magnitudes"]["value"]]
    pts = []
    for i in range(7):
        mid = (mags[i] + mags[i + 1]) / 2
        m32 = np.float32(float(mid))
        pts += [m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(10))]
    pts = np.array(pts + [np.float32(m) for m in FACTS["e2m1_magnitudes"]["value"]], np.float32)
    got = orc.e2m1_encode_rn(pts)
    for v, c in zip(pts, got):
        fv = Fraction(float(v))
        dists = [abs(fv - m) for m in mags]
        best = min(dists)
        cands = [i for i, d in enumerate(dists) if d == best]
        want = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
        assert c == want, (float(v), c, want)
    neg = orc.e2m1_encode_rn(-pts)
    assert np.array_equal(neg, got | 8)


def test_e2m1_sr_grid_points_do_not_move(orc):
    k = np.arange(65536, dtype=np.uint16)
    for c in range(8):
        v = np.full(65536, orc.e2m1_decode([c])[0], np.float32)
        assert np.all(orc.e2m1_encode_sr(v, k) == c)
        assert np.all(orc.e2m1_encode_sr(-v, k) == (c | 8))


def test_e2m1_sr_probability_matches_position(orc):
    """Over all 2^16 random integers, the share that rounds up equals the value's
    position between its neighbours to within 2^-17 (the 16-bit resolution)."""
    k = np.arange(65536, dtype=np.uint16)
    rng = np.random.default_rng(5)
    vals = rng.random(300, dtype=np.float32) * np.float32(6.0)
    mags = np.array(FACTS["e2m1_magnitudes"]["value"])
    for v in vals:
        q = orc.e2m1_encode_sr(np.full(65536, v, np.float32), k)
        lo = np.searchsorted(mags, float(v), side="right") - 1
        hi = lo + 1
        frac = (float(v) - mags[lo]) / (mags[hi] - mags[lo])
        assert set(np.unique(q)) <= {lo, hi}
        p_up = np.mean(q == hi)
        assert abs(p_up - frac) <= 2.0 ** -17 + 1e-12, (v, p_up, frac)


def test_e2m1_sr_example_thirty_percent(orc):
    """PR: 0.3 on a {0, 1} grid rounds up 30 % of the time.  E2M1's neighbours 2 and 3
    form a step-1 grid, so 2.3 must round to 3 with probability 0.3; 0.15 sits at the
    same position between 0 and 0.5.  10^6 Philox draws, |f - 0.3| < 5 sigma."""
    f = FACTS["stochastic_rounding_example"]
    n = 1_000_000
    bits = orc.sr_bits(seed=1234, first=0, n=n)
    sigma = np.sqrt(f["p_up"] * (1 - f["p_up"]) / n)
    for v, up_code in ((2.0 + f["value"], 5), (0.5 * f["value"], 1)):
        q = orc.e2m1_encode_sr(np.full(n, v, np.float32), bits)
        frac_up = np.mean(q == up_code)
        assert abs(frac_up - f["p_up"]) < 5 * sigma, (v, frac_up)


# ------------------------------------------------------------------ E4M3
def test_e4m3_decode_matches_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all(both_nan | (ours == ref))
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert ours[0x7E] == 448.0 and ours[1] == 2.0 ** -9


def test_e4m3_format_bits(orc):
    """4 exponent bits, 3 mantissa bits: 8 mantissa steps per binade, 15 binades + subnormals."""
    f = FACTS["e4m3_bits"]
    vals = orc.e4m3_decode(np.arange(127, dtype=np.uint8)).astype(np.float64)
    assert np.all(np.diff(vals) > 0)
    per_binade = 2 ** f["mantissa_bits"]
    for e in range(1, 2 ** f["exponent_bits"]):
        seg = vals[e * per_binade:(e + 1) * per_binade]
        if seg.size == per_binade:
            assert np.allclose(seg / seg[0], 1 + np.arange(per_binade) / per_binade)


def test_e4m3_encode_exhaustive_vs_torch(orc):
    """Every binary32 in [2^-11, 464] (166 M values) against torch's E4M3 cast (RNE);
    everything below 2^-11 encodes to 0."""
    a = f32_range(2.0 ** -11, 464.0)
    step = 1 << 23
    for i in range(0, a.size, step):
        chunk = a[i:i + step]
        ref = torch.from_numpy(chunk).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(orc.e4m3_encode(chunk), ref), i
    tiny = f32_range(0.0, 2.0 ** -11)[:: 997]
    assert np.all(orc.e4m3_encode(tiny) == 0)


def test_e4m3_encode_saturates(orc):
    """Above 464 torch returns NaN; the block-scale encoder saturates to 448 (code 0x7E)."""
    v = np.array([464.00003, 500.0, 1e6, 3.4e38, np.inf], np.float32)
    assert np.all(orc.e4m3_encode(v) == 0x7E)


# ------------------------------------------------------------------ bf16
def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    x = np.concatenate([x, np.array([0.0, -0.0, 1e-40, 3.3e38, 1.00390625, 1.01171875], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.f32_to_bf16(x), ref)
    y = orc.dequantize_bf16(np.zeros((16, 8), np.uint8), np.zeros((16, 1), np.uint8), 1.0, 16, 16)
    assert np.all(y == 0)


def _bf16_dequant_cases():
    """Codes 0..15 in every row, one E4M3 scale byte per row (all 256: zero, subnormals,
    both signs, 448, the NaN bytes), times tensor scales chosen so that the binary32 values
    land on bf16 ties (1 + 2^-8 goes down to even, 1 + 3 * 2^-8 up), next to them, in the
    binary32 subnormal range, at the top of the range (rounding to inf), on inf and NaN,
    and at random over 2^-140 .. 2^120."""
    codes = np.tile(np.array([(2 * j + 1) << 4 | (2 * j) for j in range(8)], np.uint8), (256, 1))
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    bits = [0x3F800000, 0x3F808000, 0x3F818000, 0x3F804000, 0x3F80C000, 0x3F7F8000,
            0x3FFF8000, 0x00018000, 0x00008000, 0x00000001, 0x00800000, 0x0B808000,
            0x7F7FFFFF, 0x7F7F8000, 0x7F000000, 0x7F800000, 0x7FC00000, 0x00000000,
            0x80000000, 0xBF808000]
    rng = np.random.default_rng(11)
    rnd = (rng.integers(-140, 120, 300).astype(np.float64) +
           rng.uniform(0, 1, 300)).astype(np.float64)
    r32 = np.exp2(rnd).astype(np.float32).view(np.uint32)
    r32 = np.concatenate([r32, (r32 & 0xFFFF0000) | 0x8000])   # and their tie patterns
    g = np.concatenate([np.array(bits, np.uint32), r32]).view(np.float32)
    return codes, scales, g


def bf16_dequant_mismatches(orc, L=None):
    """Elements where the oracle's bf16 dequantize differs from torch's binary32 -> bf16
    cast of the oracle's binary32 dequantize (NaN must stay NaN; its payload is free)."""
    codes, scales, gs = _bf16_dequant_cases()
    bad = ties = 0
    for g in gs:
        y32 = orc.dequantize(codes, scales, g, 256, 16, L=L)
        got = orc.dequantize_bf16(codes, scales, g, 256, 16, L=L)
        ref = torch.from_numpy(y32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(y32)
        got_nan = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
        bad += int(np.count_nonzero(nan != got_nan))
        bad += int(np.count_nonzero((got != ref) & ~nan))
        ties += int(np.count_nonzero((y32.view(np.uint32) & 0xFFFF) == 0x8000))
    return bad, ties


def test_dequantize_bf16_matches_torch_cast(orc):
    """The bf16 dequantize ([PR] "MVFP4与MXFP4": code value times block scale; FP32 tensor
    scale on top, "MVFP4格式的核心架构革新") equals torch's nearest-even cast of the binary32
    dequantize on every case, ties included."""
    bad, ties = bf16_dequant_mismatches(orc)
    assert bad == 0
    assert ties > 10000   # the cases do exercise the tie rule


def test_dequantize_bf16_pin_catches_round_half_up(orc, tmp_path):
    """Plant round-half-up in a copy of the oracle's bf16 conversion: the pin above fails."""
    import ctypes
    import subprocess
    src = open(os.path.join(os.path.dirname(orc.__file__), "nvfp4_oracle.c")).read()
    rne = "return (uint16_t)((u + 0x7FFFu + lsb) >> 16);"
    assert src.count(rne) == 1
    (tmp_path / "planted.c").write_text(src.replace(rne, "(void)lsb; return (uint16_t)((u + 0x8000u) >> 16);"))
    so = str(tmp_path / "planted.so")
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC",
                           "-shared", "-I", os.path.dirname(orc.__file__), "-o", so,
                           str(tmp_path / "planted.c"), "-lm"])
    planted = orc.declare(ctypes.CDLL(so))
    bad, _ = bf16_dequant_mismatches(orc, L=planted)
    assert bad > 0
