"""The hardware conversions the kernels rely on, against the oracle's codecs (GPU).

The quantizers, the dequantizers and the GEMM epilogues use gfx950's conversion
instructions through the library's device helpers (csrc/nvfp4_device.hpp); bit-exact parity
of codes and scales rests on those conversions rounding exactly as the format needs (E4M3
block scales, E2M1 elements: [NV-blog] recipe section, bullets 1-2; [PR]
"MVFP4格式的核心架构革新").  tests/native/conv_probe.hip runs the helpers themselves over
large input sets; each result is compared with the CPU oracle:

* e4m3_encode (clamp at 448 + fp8 conversion) on every binary32 in [0, 464] (and a sweep
  above, up to inf) against ``orc_e4m3_encode``;
* e2m1_rn_pack16 (scaled fp4 conversion, scale 1.0) on every binary32 in [0, 8], every
  13th pattern of the negative range down to -inf, and a sweep above 8 against
  ``orc_e2m1_encode_rn``;
* bf16_bits_rn (the GEMM epilogues' fp32 -> bf16) on all 2^32 binary32 patterns against
  ``orc_f32_to_bf16`` (itself pinned against torch's cast), NaN compared as NaN;
* the decoders (fp8 -> fp32 and fp16, fp4 -> fp32, the GEMM's fp4 x scale -> fp16) on
  every code against ``orc_e4m3_decode`` / ``orc_e2m1_decode`` and their exact product;
* e2m1_sr_pack16, the stochastic encoder on the hardware stochastic fp4 conversion, against
  ``orc_e2m1_encode_sr`` at every decision point of every 16-bit draw (the exact point,
  one and two ulps and fractions of a 2^-23 unit on either side, in every grid cell, both
  signs) and on a sweep of [0, 8) with random draws ([NV-blog] recipe section bullet 5;
  [PR] outliers section: a value rounds up with probability equal to its position);
* the fp4 -> fp16 conversion's own scale operand: it applies only the power of two of the
  scale (1.5 acts as 1, 3 as 2, 448 as 256), which is why the GEMM converts with scale 1.0
  and multiplies by the E4M3 block scale in a separate packed fp16 product.

The probe is built by ``__graft_entry__.build()``; a GPU run without it fails.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "tests", "native", "libconv_probe.so")
CHUNK = 1 << 27


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(PROBE):
        pytest.fail("tests/native/libconv_probe.so is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(PROBE)
    u32, u64, P = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p
    for name in ("probe_e4m3_encode", "probe_e2m1_encode", "probe_bf16"):
        getattr(L, name).argtypes = [u32, u32, u64, P, P]
        getattr(L, name).restype = ctypes.c_int
    L.probe_e2m1_sr.argtypes = [P, P, u64, P, P]
    L.probe_e2m1_sr.restype = ctypes.c_int
    L.probe_tables.argtypes = [P, P, P, P, P, P]
    L.probe_tables.restype = ctypes.c_int
    L.probe_scale_operand.argtypes = [P, u32, P, P]
    L.probe_scale_operand.restype = ctypes.c_int
    return L


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _patterns(first, stride, n):
    """binary32 values with bit patterns first + i * stride (mod 2^32), i < n <= 2^32 - 1."""
    i = np.arange(n, dtype=np.uint32)
    i *= np.uint32(stride)
    i += np.uint32(first)
    return i.view(np.float32)


def _ranges(lo_bits, hi_bits, stride=1):
    """(first, stride, n) chunks covering the patterns lo_bits .. hi_bits inclusive."""
    total = (hi_bits - lo_bits) // stride + 1
    step = CHUNK
    for k in range(0, total, step):
        yield lo_bits + k * stride, stride, min(step, total - k)


def test_e4m3_encode_matches_oracle(probe):
    out = torch.empty(CHUNK, dtype=torch.uint8, device="cuda")
    # every binary32 in [0, 464] (464.0 = 0x43E80000), every 4099th pattern above, and inf
    ranges = (list(_ranges(0, 0x43E80000)) + list(_ranges(0x43E80000, 0x7F7FFFFF, 4099))
              + [(0x7F800000, 0, 1)])
    checked = 0
    for first, stride, n in ranges:
        print("e4m3 chunk 0x%08x stride %d n %d" % (first, stride, n), flush=True)
        assert probe.probe_e4m3_encode(first, stride, n, ctypes.c_void_p(out.data_ptr()),
                                       _stream()) == 0
        got = out[:n].cpu().numpy()
        ref = oracle.e4m3_encode(_patterns(first, stride, n))
        bad = np.flatnonzero(got != ref)
        assert bad.size == 0, "first mismatch at pattern 0x%08x: %d vs %d" % (
            (first + int(bad[0]) * stride) & 0xFFFFFFFF, got[bad[0]], ref[bad[0]])
        checked += n
    assert checked > 0x43E80000


def _pack(codes):
    c = codes.reshape(-1, 2)
    return (c[:, 0] | (c[:, 1] << 4)).astype(np.uint8)


def test_e2m1_encode_matches_oracle(probe):
    out = torch.empty(CHUNK // 2, dtype=torch.uint8, device="cuda")
    ranges = (list(_ranges(0, 0x41000000 + 15))                # [0, 8] (8.0 = 0x41000000)
              + list(_ranges(0x41000000, 0x7F7FFFFF, 4099))     # above 8, every 4099th
              + list(_ranges(0x80000000, 0xFF7FFFFF, 13))       # negatives, every 13th
              + [(0x7F800000, 0, 16), (0xFF800000, 0, 16)])     # +-inf
    for first, stride, n in ranges:
        n -= n % 16
        if n == 0:
            continue
        print("e2m1 chunk 0x%08x stride %d n %d" % (first, stride, n), flush=True)
        assert probe.probe_e2m1_encode(first, stride, n // 16, ctypes.c_void_p(out.data_ptr()),
                                       _stream()) == 0
        got = out[:n // 2].cpu().numpy()
        ref = _pack(oracle.e2m1_encode_rn(_patterns(first, stride, n)))
        bad = np.flatnonzero(got != ref)
        assert bad.size == 0, "first mismatch in byte %d of chunk 0x%08x: %02x vs %02x" % (
            bad[0], first, got[bad[0]], ref[bad[0]])


def test_bf16_conversion_matches_oracle_on_every_binary32(probe):
    out = torch.empty(CHUNK, dtype=torch.int16, device="cuda")
    nan_count = 0
    for first, stride, n in _ranges(0, 0xFFFFFFFF):
        print("bf16 chunk 0x%08x n %d" % (first, n), flush=True)
        assert probe.probe_bf16(first, stride, n, ctypes.c_void_p(out.data_ptr()),
                                _stream()) == 0
        got = out[:n].cpu().numpy().view(np.uint16)
        f = _patterns(first, stride, n)
        ref = oracle.f32_to_bf16(f)
        nan = np.isnan(f)
        got_nan = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
        assert np.array_equal(got_nan, nan), "NaN handling differs in chunk 0x%08x" % first
        bad = np.flatnonzero((got != ref) & ~nan)
        assert bad.size == 0, "first mismatch at pattern 0x%08x" % (first + int(bad[0]))
        nan_count += int(nan.sum())
    assert nan_count == 2 * (0x7FFFFF)   # both signs, every nonzero mantissa


def test_decoders_match_oracle(probe):
    e4 = torch.empty(256, dtype=torch.float32, device="cuda")
    e2 = torch.empty(512, dtype=torch.float32, device="cuda")
    sp = torch.empty(65536, dtype=torch.int32, device="cuda")      # packed fp16 pairs
    dq = torch.empty(4096 * 8, dtype=torch.int16, device="cuda")   # 8 fp16 per (scale, code)
    mm = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert probe.probe_tables(*(ctypes.c_void_p(t.data_ptr()) for t in (e4, e2, sp, dq, mm)),
                              _stream()) == 0
    torch.cuda.synchronize()
    assert mm.item() == 0, "a byte position or register half decodes differently: %d" % mm.item()
    codes = np.arange(256, dtype=np.uint8)
    ref4 = oracle.e4m3_decode(codes)
    got4 = e4.cpu().numpy()
    nan = np.isnan(ref4)
    assert np.array_equal(np.isnan(got4), nan)
    assert np.array_equal(got4[~nan].view(np.uint32), ref4[~nan].view(np.uint32))
    # fp4 pairs: byte t -> (code t & 15, code t >> 4)
    ref2 = oracle.e2m1_decode(np.stack([codes & 15, codes >> 4], 1).ravel())
    assert np.array_equal(e2.cpu().numpy().view(np.uint32), ref2.view(np.uint32))
    # E4M3 byte pairs as fp16: byte b0 of pair p in the low half, b1 in the high half
    got_sp = sp.cpu().numpy().view(np.uint32)
    got_sp = np.stack([got_sp & 0xFFFF, got_sp >> 16], 1).astype(np.uint16).view(
        np.float16).astype(np.float64)
    p = np.arange(65536)
    for h, b in ((0, p & 0xFF), (1, p >> 8)):
        ref = oracle.e4m3_decode(b.astype(np.uint8)).astype(np.float64)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got_sp[:, h]), nan)
        assert np.array_equal(got_sp[~nan, h], ref[~nan])
        # signed zeros keep their sign
        assert np.array_equal(np.signbit(got_sp[~nan, h]), np.signbit(ref[~nan]))
    # the GEMM's operand values: e2m1(c) * e4m3(s) in fp16, exact for every finite scale
    # (all eight positions of the dword hold the same code, so all eight values agree)
    got_dq = dq.cpu().numpy().view(np.float16).astype(np.float64).reshape(256, 16, 8)
    ref_dq = (oracle.e4m3_decode(codes).astype(np.float64)[:, None] *
              oracle.e2m1_decode(np.arange(16, dtype=np.uint8)).astype(np.float64)[None, :])
    ref_dq = np.repeat(ref_dq[:, :, None], 8, axis=2)
    nan = np.isnan(ref_dq)
    assert np.array_equal(np.isnan(got_dq), nan)
    assert np.array_equal(got_dq[~nan], ref_dq[~nan])


def _sr_decision_cases():
    """(values, draws): every decision point lo + (2k + 1) step 2^-17 of every draw k in
    every grid cell, with 1 and 2 ulps and sub-2^-23 offsets on either side (values below 1
    have finer ulps than the 2^-23 grid the encoder rounds up to), a sweep of [0, 8) with
    random draws, zeros, saturating values; then all of them negated."""
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4], np.float64)
    step = np.array([.5, .5, .5, .5, 1, 1, 2], np.float64)
    k = np.arange(65536, dtype=np.float64)
    vs, ks = [], []
    for lo, st in zip(grid, step):
        t = lo + (2 * k + 1) * st * 2.0 ** -17
        t32 = t.astype(np.float32)
        assert np.all(t32.astype(np.float64) == t)   # the decision points are binary32
        x = t32
        for d in range(3):
            up, dn = x.copy(), x.copy()
            for _ in range(d):
                up = np.nextafter(up, np.float32(np.inf))
                dn = np.nextafter(dn, np.float32(-np.inf))
            vs += [up, dn] if d else [x]
            ks += [np.arange(65536, dtype=np.uint16)] * (2 if d else 1)
        for off in (2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26):
            for sgn in (-1, 1):
                vs.append((t + sgn * off).astype(np.float32))
                ks.append(np.arange(65536, dtype=np.uint16))
    rng = np.random.default_rng(3)
    sweep = np.arange(0, 0x41000000, 997, dtype=np.uint32).view(np.float32)
    vs.append(sweep)
    ks.append(rng.integers(0, 65536, sweep.size).astype(np.uint16))
    vs.append(np.array([0.0, 6.0, 7.9, 100.0, 1e-30, 2.0 ** -18, 2.0 ** -19, 0.25], np.float32))
    ks.append(np.array([0, 1, 2, 3, 4, 0, 65535, 32767], np.uint16))
    v = np.concatenate(vs)
    kk = np.concatenate(ks)
    v, kk = np.concatenate([v, -v]), np.concatenate([kk, kk])
    n = v.size - v.size % 16
    return np.ascontiguousarray(v[:n]), np.ascontiguousarray(kk[:n])


def test_stochastic_encoder_matches_oracle_at_every_decision_point(probe):
    v, k = _sr_decision_cases()
    n16 = v.size // 16
    print("stochastic encoder: %d values" % v.size, flush=True)
    tv = torch.from_numpy(v).cuda()
    tk = torch.from_numpy(k.view(np.int16)).cuda()
    out = torch.empty(n16 * 8, dtype=torch.uint8, device="cuda")
    assert probe.probe_e2m1_sr(ctypes.c_void_p(tv.data_ptr()), ctypes.c_void_p(tk.data_ptr()),
                               n16, ctypes.c_void_p(out.data_ptr()), _stream()) == 0
    got = out.cpu().numpy()
    ref = _pack(oracle.e2m1_encode_sr(v, k))
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, "%d bytes differ; first: value %r draw %d, gpu %02x oracle %02x" % (
        bad.size, float(v[2 * bad[0]]), k[2 * bad[0]], got[bad[0]], ref[bad[0]])


def test_fp4_conversion_scale_operand_applies_only_its_power_of_two(probe):
    # every code, in all eight positions, converted with scales that carry a mantissa: the
    # result is the code's value times 2^floor(log2 scale), not times the scale
    scales = np.array([1.0, 1.25, 1.5, 1.875, 2.0, 3.0, 0.375, 448.0, 0.125, 6.0, 1.5 * 2.0 ** -9],
                      dtype=np.float32)
    s = torch.from_numpy(scales).cuda()
    out = torch.empty(16 * len(scales) * 16, dtype=torch.uint8, device="cuda")
    assert probe.probe_scale_operand(s.data_ptr(), len(scales), out.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.float16).reshape(len(scales), 16, 8).astype(np.float64)
    codes = np.arange(16)
    val = oracle.e2m1_decode(codes).astype(np.float64)
    for k, sc in enumerate(scales):
        p2 = 2.0 ** np.floor(np.log2(np.float64(sc)))
        want = np.repeat((val * p2)[:, None], 8, axis=1)
        assert np.array_equal(got[k], want), (sc, got[k][:, 0], want[:, 0])
