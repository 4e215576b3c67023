// dequantize.hip -- NVFP4 -> bf16 / fp32 for gfx950.
//
// y = (e2m1(code) * e4m3(scale)) * global: a stored 4-bit value times its block scale is
// the real value (prism.simon-ai.net article 7890, section "MVFP4与MXFP4：通过缩放实现低精度推理":
// 6 with a block scale of 100 is 600), with the FP32 tensor scale on top (section
// "MVFP4格式的核心架构革新").  The first product is exact in binary32; the second rounds
// once; bf16 output rounds that to nearest-even.
//
// One thread per 16-element row group: one 8-byte code load, one scale byte, and 32 or
// 64 bytes of 16-byte stores.  The kernel is HBM-bound (9 bytes in, 32 or 64 out per 16
// elements).
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Byte B of w holds two E2M1 codes (low nibble first): decode both to fp32 with the
// hardware conversion (scale 1.0, exact), then (e2m1 * sbd) * s.
template <int B>
__device__ __forceinline__ void decode_byte(uint32_t w, float sbd, float s, float *v) {
  const float2_t f = e2m1_decode_pair<B>(w);
  v[0] = (f[0] * sbd) * s;   // first product exact
  v[1] = (f[1] * sbd) * s;
}

template <bool F32, bool B16>
__global__ __launch_bounds__(kThreads) void dequant_kernel(
    const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
    const float *__restrict__ global_dec, uint32_t ngroups, uint32_t gpr, int64_t ld_y,
    void *__restrict__ y) {
  const float s = *global_dec;
  for (uint32_t g = blockIdx.x * kThreads + threadIdx.x; g < ngroups;
       g += gridDim.x * kThreads) {
    const uint32_t r = g / gpr, gc = g - r * gpr;
    const uint2 cw = reinterpret_cast<const uint2 *>(codes)[g];
    const uint32_t sidx = B16 ? (r >> 4) * gpr + gc : g;
    const float sbd = e4m3_decode(scales[sidx]);
    float v[16];
    decode_byte<0>(cw.x, sbd, s, v + 0);
    decode_byte<1>(cw.x, sbd, s, v + 2);
    decode_byte<2>(cw.x, sbd, s, v + 4);
    decode_byte<3>(cw.x, sbd, s, v + 6);
    decode_byte<0>(cw.y, sbd, s, v + 8);
    decode_byte<1>(cw.y, sbd, s, v + 10);
    decode_byte<2>(cw.y, sbd, s, v + 12);
    decode_byte<3>(cw.y, sbd, s, v + 14);
    const size_t off = (size_t)r * (size_t)ld_y + (size_t)gc * 16u;
    if (F32) {
      float4 *dst = reinterpret_cast<float4 *>(reinterpret_cast<float *>(y) + off);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    } else {
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        h[i] = f32_to_bf16_bits(v[2 * i]) | (f32_to_bf16_bits(v[2 * i + 1]) << 16);
      uint4 *dst = reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(y) + off);
      dst[0] = make_uint4(h[0], h[1], h[2], h[3]);
      dst[1] = make_uint4(h[4], h[5], h[6], h[7]);
    }
  }
}

}  // namespace

hipError_t launch_dequantize(const DequantLaunch &d, hipStream_t stream) {
  const uint64_t ngroups = (uint64_t)d.rows * (uint64_t)(d.cols / 16);
  if (ngroups == 0) return hipSuccess;
  uint64_t grid = (ngroups + kThreads - 1) / kThreads;
  if (grid > 8192) grid = 8192;
  const uint32_t gpr = (uint32_t)(d.cols / 16);
#define NVFP4_DQ(F, B)                                                                     \
  dequant_kernel<F, B><<<(uint32_t)grid, kThreads, 0, stream>>>(                           \
      d.codes, d.scales, d.global_dec, (uint32_t)ngroups, gpr, d.ld_y, d.y)
  if (d.out_f32) { if (d.blocking) NVFP4_DQ(true, true); else NVFP4_DQ(true, false); }
  else { if (d.blocking) NVFP4_DQ(false, true); else NVFP4_DQ(false, false); }
#undef NVFP4_DQ
  return hipGetLastError();
}

}  // namespace nvfp4
