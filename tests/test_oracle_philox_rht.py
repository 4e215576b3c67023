"""Pins for the oracle's Philox4x32-10 stream and 16-point random Hadamard transform.

Philox: compared with rocRAND's host implementation of Philox4x32-10 (a library
routine, compiled here from its header), plus uniformity and the element-to-bit map.
RHT: compared with scipy's Sylvester Hadamard matrix in binary64, and against the
closed forms the transform must satisfy (norm and dot products kept, as the prism
article's section on outliers and rounding states; unit and constant vectors).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
import scipy.linalg

ROCRAND_PROBE = r"""
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
struct Engine : rocrand_device::philox4x32_10_engine {
  using rocrand_device::philox4x32_10_engine::ten_rounds;
};
int main() {
  unsigned k0, k1, c0, c1, c2, c3;
  Engine e;
  while (scanf("%x %x %x %x %x %x", &k0, &k1, &c0, &c1, &c2, &c3) == 6) {
    uint4 r = e.ten_rounds(uint4{c0, c1, c2, c3}, uint2{k0, k1});
    printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists(
            "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc / rocRAND headers not available")
    d = tmp_path_factory.mktemp("philox")
    src = d / "probe.cpp"
    src.write_text(ROCRAND_PROBE)
    exe = d / "probe"
    subprocess.check_call([hipcc, "-O1", str(src), "-o", str(exe)],
                          stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)

    def run(key, ctr):
        lines = "".join("%x %x %x %x %x %x\n" % (k[0], k[1], c[0], c[1], c[2], c[3])
                        for k, c in zip(key, ctr))
        out = subprocess.run([str(exe)], input=lines, capture_output=True, text=True,
                             check=True).stdout.split()
        return np.array([int(v, 16) for v in out], dtype=np.uint32).reshape(-1, 4)
    return run


def test_philox_matches_rocrand(orc, rocrand_philox):
    rng = np.random.default_rng(99)
    n = 2000
    ctr = rng.integers(0, 2 ** 32, (n, 4), dtype=np.uint32)
    key = rng.integers(0, 2 ** 32, (n, 2), dtype=np.uint32)
    ctr[0] = 0
    key[0] = 0
    ctr[1] = 0xFFFFFFFF
    key[1] = 0xFFFFFFFF
    ours = orc.philox4x32_10(ctr, key)
    ref = rocrand_philox(key, ctr)
    assert np.array_equal(ours, ref)


def test_philox_uniformity(orc):
    """Chi-square of the 16-bit SR draws (top and bottom byte, 256 bins each) over 2^22
    consecutive element indices; threshold = chi2 quantile 1 - 1e-6 (df 255)."""
    from scipy.stats import chi2
    bits = orc.sr_bits(seed=0xC0FFEE, first=0, n=1 << 22)
    lim = chi2.ppf(1 - 1e-6, 255)
    for part in (bits >> 8, bits & 0xFF):
        h = np.bincount(part.astype(np.int64), minlength=256)
        e = bits.size / 256
        assert ((h - e) ** 2 / e).sum() < lim


def test_sr_bits_layout(orc):
    """Element i takes 16-bit lane (i & 7) of the Philox block with counter i >> 3."""
    seed = 0x123456789ABCDEF
    first = 8 * 1000
    n = 64
    bits = orc.sr_bits(seed, first, n)
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint32)
    for g in range(n // 8):
        blk = orc.philox4x32_10(np.array([[first // 8 + g, 0, 0, 0]], np.uint32), key)[0]
        halves = [(int(blk[w]) >> (16 * h)) & 0xFFFF for w in range(4) for h in range(2)]
        assert list(bits[8 * g:8 * g + 8]) == halves
    # counter-based: any sub-range equals the matching slice of a longer draw
    assert np.array_equal(orc.sr_bits(seed, first + 24, 16), bits[24:40])


# ------------------------------------------------------------------ RHT
def test_rht_signs(orc):
    d = orc.rht_signs(0x5248)
    assert set(np.unique(d)) <= {-1.0, 1.0}
    assert np.array_equal(d, orc.rht_signs(0x5248))
    assert not np.array_equal(d, orc.rht_signs(0x5249))
    key = np.array([0x5248, 0], np.uint32)
    w = orc.philox4x32_10(np.array([[0, 0, 1, 0]], np.uint32), key)[0, 0]
    assert np.array_equal(d, np.where((int(w) >> np.arange(16)) & 1, -1.0, 1.0))


def test_rht_matches_scipy_hadamard(orc):
    H = scipy.linalg.hadamard(16).astype(np.float64)
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((4096, 16)) * np.exp(rng.uniform(-5, 5, (4096, 1)))).astype(np.float32)
    d = orc.rht_signs(0x5248).astype(np.float64)
    y = orc.rht16(x.ravel(), 0x5248).reshape(-1, 16).astype(np.float64)
    y64 = 0.25 * (x.astype(np.float64) * d) @ H.T
    bound = 4 * 2.0 ** -24 * np.abs(x).astype(np.float64).sum(1, keepdims=True)
    assert np.all(np.abs(y - y64) <= bound)


def test_rht_keeps_norm_and_dot_products(orc):
    rng = np.random.default_rng(1)
    a = rng.standard_normal(16 * 10000).astype(np.float32)
    b = rng.standard_normal(16 * 10000).astype(np.float32)
    ya = orc.rht16(a, 7).astype(np.float64).reshape(-1, 16)
    yb = orc.rht16(b, 7).astype(np.float64).reshape(-1, 16)
    a64, b64 = a.astype(np.float64).reshape(-1, 16), b.astype(np.float64).reshape(-1, 16)
    na, nya = np.linalg.norm(a64, axis=1), np.linalg.norm(ya, axis=1)
    assert np.all(np.abs(nya - na) <= 1e-6 * na)
    dots, ydots = (a64 * b64).sum(1), (ya * yb).sum(1)
    assert np.all(np.abs(ydots - dots) <= 1e-6 * na * np.linalg.norm(b64, axis=1))


def test_rht_closed_forms(orc):
    ones = np.ones(16, np.float32)
    # constant vector with all signs +1 -> (4c, 0, ..., 0), exactly
    c = np.float32(0.8125)
    y = orc.rht16_with_signs(np.full(16, c, np.float32), ones)
    assert y[0] == 4 * c and np.all(y[1:] == 0)
    # unit vectors -> +-1/4 with the Sylvester sign pattern H[i][j] = (-1)^popcount(i & j)
    d = orc.rht_signs(3)
    for j in range(16):
        e = np.zeros(16, np.float32)
        e[j] = 1
        y = orc.rht16_with_signs(e, d)
        want = np.array([d[j] * 0.25 * (-1) ** bin(i & j).count("1") for i in range(16)], np.float32)
        assert np.array_equal(y, want)
    # involution: applying the unsigned transform again and the signs returns x
    rng = np.random.default_rng(2)
    x = rng.standard_normal(16 * 100).astype(np.float32)
    y = orc.rht16_with_signs(x, d)
    back = orc.rht16_with_signs(y, ones).reshape(-1, 16) * 4 * 0.25 * d
    assert np.allclose(back.ravel(), x, rtol=0, atol=1e-6 * np.abs(x).max())
