// conv_probe.hip -- test-only kernels that run the library's device conversion helpers
// (block_scaled_fp4_06_amd/csrc/nvfp4_device.hpp) over large sets of inputs, so that the
// GPU tests can compare them with the CPU oracle's codecs value by value.
//
// The quantizers and the GEMM rely on these hardware conversions being exactly the
// rounding the pages' format needs (E4M3 block scales and E2M1 elements, [NV-blog]
// recipe section bullets 1-2; [PR] "MVFP4格式的核心架构革新"):
//   e4m3_encode       clamp at 448, then the fp8 conversion: nearest-even E4M3FN code;
//   e4m3_decode       fp8 -> fp32;  e4m3_pair_f16: fp8 -> fp16 (the GEMM's block scales);
//   e2m1_rn_pack16    the scaled fp4 conversion with scale 1.0: nearest-even E2M1 codes;
//   e2m1_decode_pair  fp4 -> fp32;  dequant8_f16: fp4 -> fp16 times the block scale;
//   bf16_bits_rn      fp32 -> bf16 nearest-even (the GEMM epilogues);
//   e2m1_sr_pack16    the stochastic E2M1 encoder on the hardware stochastic fp4 conversion;
//   and the fp4 -> fp16 conversion's own scale operand, which the GEMM leaves at 1.0.
// Inputs are generated on the device from binary32 bit patterns first + i * stride
// (modulo 2^32); every entry point launches on the caller's stream and returns the HIP
// status of the launch.  Grids are grid-stride loops over exactly n items.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_device.hpp"

namespace {

constexpr int kThreads = 256;

unsigned grid_for(uint64_t n) {
  const uint64_t g = (n + kThreads - 1) / kThreads;
  return (unsigned)(g < 16384 ? (g ? g : 1) : 16384);
}

__device__ __forceinline__ float pattern(uint32_t first, uint32_t stride, uint64_t i) {
  return __uint_as_float(first + (uint32_t)i * stride);
}

__global__ void e4m3_encode_kernel(uint32_t first, uint32_t stride, uint64_t n, uint8_t *out) {
  for (uint64_t i = blockIdx.x * (uint64_t)kThreads + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * kThreads)
    out[i] = (uint8_t)nvfp4::e4m3_encode(pattern(first, stride, i));
}

// n16 groups of 16 consecutive patterns, each packed to 8 bytes of codes (multiplier 1.0)
__global__ void e2m1_encode_kernel(uint32_t first, uint32_t stride, uint64_t n16, uint2 *out) {
  for (uint64_t g = blockIdx.x * (uint64_t)kThreads + threadIdx.x; g < n16;
       g += (uint64_t)gridDim.x * kThreads) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = pattern(first, stride, 16 * g + j);
    out[g] = nvfp4::e2m1_rn_pack16(v, 1.0f);
  }
}

__global__ void bf16_kernel(uint32_t first, uint32_t stride, uint64_t n, uint16_t *out) {
  for (uint64_t i = blockIdx.x * (uint64_t)kThreads + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * kThreads)
    out[i] = nvfp4::bf16_bits_rn(pattern(first, stride, i));
}

// n16 groups of 16 host-given values v with 16-bit draws k: the stochastic codes of
// e2m1_sr_pack16, whose input is v * 2^23 and whose draw words hold element 2i's draw in
// the low and element 2i+1's in the high half of word i.
__global__ void e2m1_sr_kernel(const float *v, const uint16_t *k, uint64_t n16, uint2 *out) {
  for (uint64_t g = blockIdx.x * (uint64_t)kThreads + threadIdx.x; g < n16;
       g += (uint64_t)gridDim.x * kThreads) {
    float t[16];
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 16; ++j) t[j] = v[16 * g + j] * 0x1p23f;
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = k[16 * g + 2 * i] | ((uint32_t)k[16 * g + 2 * i + 1] << 16);
    out[g] = nvfp4::e2m1_sr_pack16(t, w);
  }
}

// Small tables, one thread per entry:
//   e4m3_dec[c]          e4m3_decode(c) for every byte c                     (256 floats)
//   e2m1_dec[2 t + h]    e2m1_decode_pair of byte t: h = 0 the low nibble, 1 the high one
//                        (512 floats); the byte in positions 1-3 must decode alike
//                        (else bit 0 of *mismatch)
//   scale_pairs[p]       e4m3_pair_f16 of the byte pair p = b1 << 8 | b0, as the packed
//                        register (low fp16 = b0, high = b1; 65536 dwords); the pair in the
//                        upper half of the word must decode alike (else bit 1)
//   dequant[8 (16 s + c) + j]  element j of dequant8_f16(code c in all eight positions,
//                        scale = e4m3 byte s as fp16), stored as the four packed registers
//                        (4096 x 8 fp16)
// Results are stored as whole packed registers: this compiler stores the low half of the
// register for an fp16 element taken out of a packed conversion result on its own.
__global__ void tables_kernel(float *e4m3_dec, float *e2m1_dec, uint32_t *scale_pairs,
                              uint4 *dequant, uint32_t *mismatch) {
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  if (t < 256u) e4m3_dec[t] = nvfp4::e4m3_decode(t);
  if (t < 256u) {
    // byte position b (0..3) holding the code pair (lo = t & 15, hi = t >> 4)
    const uint32_t byte = t & 0xFFu;
    const nvfp4::float2_t p0 = nvfp4::e2m1_decode_pair<0>(byte);
    const nvfp4::float2_t p1 = nvfp4::e2m1_decode_pair<1>(byte << 8);
    const nvfp4::float2_t p2 = nvfp4::e2m1_decode_pair<2>(byte << 16);
    const nvfp4::float2_t p3 = nvfp4::e2m1_decode_pair<3>(byte << 24);
    // every position must decode alike; store position 0 and flag differences
    e2m1_dec[2 * t] = p0[0];
    e2m1_dec[2 * t + 1] = p0[1];
    if (__float_as_uint(p1[0]) != __float_as_uint(p0[0]) || __float_as_uint(p1[1]) != __float_as_uint(p0[1]) ||
        __float_as_uint(p2[0]) != __float_as_uint(p0[0]) || __float_as_uint(p2[1]) != __float_as_uint(p0[1]) ||
        __float_as_uint(p3[0]) != __float_as_uint(p0[0]) || __float_as_uint(p3[1]) != __float_as_uint(p0[1]))
      atomicOr(mismatch, 1u);
  }
  if (t < 65536u) {
    const uint32_t lo = __builtin_bit_cast(uint32_t, nvfp4::e4m3_pair_f16(t, 0));
    const uint32_t hi = __builtin_bit_cast(uint32_t, nvfp4::e4m3_pair_f16(t << 16, 1));
    scale_pairs[t] = lo;
    if (hi != lo) atomicOr(mismatch, 2u);
  }
  if (t < 4096u) {
    const uint32_t s = t >> 4, c = t & 15u;
    const _Float16 sbd = nvfp4::e4m3_pair_f16(s, 0).x;
    const uint32_t w = c * 0x11111111u;   // the code in all eight positions
    dequant[t] = __builtin_bit_cast(uint4, nvfp4::dequant8_f16(w, sbd));
  }
}

// The fp4 -> fp16 conversion with a scale operand other than 1.0: code c in all eight
// positions of a dword, converted with scale s[k]; out[16 k + c] holds the four packed
// result registers (8 fp16).  One thread per (k, c); n = 16 * number of scales.
__global__ void scale_operand_kernel(const float *s, uint32_t n, uint4 *out) {
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= n) return;
  const float sc = s[t >> 4];
  const uint32_t w = (t & 15u) * 0x11111111u;
  const nvfp4::half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 0);
  const nvfp4::half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 1);
  const nvfp4::half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 2);
  const nvfp4::half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 3);
  out[t] = make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                      __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
}

}  // namespace

extern "C" {

int probe_e4m3_encode(uint32_t first, uint32_t stride, uint64_t n, uint8_t *out, hipStream_t s) {
  e4m3_encode_kernel<<<grid_for(n), kThreads, 0, s>>>(first, stride, n, out);
  return (int)hipGetLastError();
}

int probe_e2m1_encode(uint32_t first, uint32_t stride, uint64_t n16, uint8_t *out, hipStream_t s) {
  e2m1_encode_kernel<<<grid_for(n16), kThreads, 0, s>>>(first, stride, n16,
                                                        reinterpret_cast<uint2 *>(out));
  return (int)hipGetLastError();
}

int probe_bf16(uint32_t first, uint32_t stride, uint64_t n, uint16_t *out, hipStream_t s) {
  bf16_kernel<<<grid_for(n), kThreads, 0, s>>>(first, stride, n, out);
  return (int)hipGetLastError();
}

int probe_e2m1_sr(const float *v, const uint16_t *k, uint64_t n16, uint8_t *out, hipStream_t s) {
  e2m1_sr_kernel<<<grid_for(n16), kThreads, 0, s>>>(v, k, n16, reinterpret_cast<uint2 *>(out));
  return (int)hipGetLastError();
}

int probe_scale_operand(const float *s, uint32_t nscales, uint8_t *out, hipStream_t st) {
  const uint32_t n = 16u * nscales;
  scale_operand_kernel<<<(n + kThreads - 1) / kThreads, kThreads, 0, st>>>(
      s, n, reinterpret_cast<uint4 *>(out));
  return (int)hipGetLastError();
}

int probe_tables(float *e4m3_dec, float *e2m1_dec, uint32_t *scale_pairs, uint4 *dequant,
                 uint32_t *mismatch, hipStream_t s) {
  tables_kernel<<<65536 / kThreads, kThreads, 0, s>>>(e4m3_dec, e2m1_dec, scale_pairs, dequant,
                                                      mismatch);
  return (int)hipGetLastError();
}

}  // extern "C"
