// dequantize.hip -- NVFP4 -> bf16 / fp32 for gfx950.
//
// y = (e2m1(code) * e4m3(scale)) * global: a stored 4-bit value times its block scale is
// the real value (prism.simon-ai.net article 7890, section "MVFP4与MXFP4：通过缩放实现低精度推理":
// 6 with a block scale of 100 is 600), with the FP32 tensor scale on top (section
// "MVFP4格式的核心架构革新").  The first product is exact in binary32; the second rounds
// once; bf16 output rounds that to nearest-even.
//
// One thread per part of a row group, 8 elements for bf16 output and 4 for fp32 (4 or 2
// code bytes in, 16 bytes out), so each store instruction of a wave writes 1 KiB of
// consecutive output, with non-temporal stores.  In the linear-layer step (quantize X,
// quantize W, GEMM, dequantize X, repeated) ordinary or write-through stores of the 84 MB
// output displace the weight from the 256 MB Infinity Cache, and the next weight quantize
// pays for it (118-119 us against 101-104 us; step 1.410 against 1.394 ms).  The kernel
// is HBM-bound (9 bytes in, 32 or 64 out per 16 elements).
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

typedef int v4i32 __attribute__((ext_vector_type(4)));

// 16 bytes at byte offset `off` of y, non-temporal: the output is written once, and a
// stream of ordinary or write-through stores would displace from the 256 MB Infinity Cache
// what the caller reads next (see the file comment).
__device__ __forceinline__ void store16(void *y, size_t off, v4i32 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<v4i32 *>(static_cast<uint8_t *>(y) + off));
}

// Part q of the output: row group q / P, elements E (q % P) .. + E - 1 of it.
template <bool F32, bool B16>
__global__ __launch_bounds__(kThreads) void dequant_kernel(
    const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
    const float *__restrict__ global_dec, uint64_t nparts, uint32_t gpr, int64_t ld_y,
    void *__restrict__ y) {
  constexpr uint32_t E = F32 ? 4 : 8, P = 16 / E;
  const float s = *global_dec;
  for (uint64_t q = (uint64_t)blockIdx.x * kThreads + threadIdx.x; q < nparts;
       q += (uint64_t)gridDim.x * kThreads) {
    const uint32_t g = (uint32_t)(q / P), part = (uint32_t)(q % P);
    const uint32_t r = g / gpr, gc = g - r * gpr;
    const uint32_t sidx = B16 ? (r >> 4) * gpr + gc : g;
    const float sbd = e4m3_decode(scales[sidx]);
    const size_t off = (size_t)r * (size_t)ld_y + (size_t)gc * 16u + part * E;
    if (F32) {
      const uint32_t cw = reinterpret_cast<const uint16_t *>(codes)[q];   // 2 code bytes
      float v[4];
      decode_byte<0>(cw, sbd, s, v + 0);
      decode_byte<1>(cw, sbd, s, v + 2);
      const v4i32 w = {(int)__float_as_uint(v[0]), (int)__float_as_uint(v[1]),
                       (int)__float_as_uint(v[2]), (int)__float_as_uint(v[3])};
      store16(y, off * 4, w);
    } else {
      const uint32_t cw = reinterpret_cast<const uint32_t *>(codes)[q];   // 4 code bytes
      float v[8];
      decode_byte<0>(cw, sbd, s, v + 0);
      decode_byte<1>(cw, sbd, s, v + 2);
      decode_byte<2>(cw, sbd, s, v + 4);
      decode_byte<3>(cw, sbd, s, v + 6);
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        h[i] = f32_to_bf16_bits(v[2 * i]) | (f32_to_bf16_bits(v[2 * i + 1]) << 16);
      store16(y, off * 2, (v4i32){(int)h[0], (int)h[1], (int)h[2], (int)h[3]});
    }
  }
}

}  // namespace

hipError_t launch_dequantize(const DequantLaunch &d, hipStream_t stream) {
  const uint64_t ngroups = (uint64_t)d.rows * (uint64_t)(d.cols / 16);
  if (ngroups == 0) return hipSuccess;
  const uint64_t nparts = ngroups * (d.out_f32 ? 4u : 2u);
  uint64_t grid = (nparts + kThreads - 1) / kThreads;
  if (grid > 16384) grid = 16384;
  const uint32_t gpr = (uint32_t)(d.cols / 16);
#define NVFP4_DQ(F, B)                                                                     \
  dequant_kernel<F, B><<<(uint32_t)grid, kThreads, 0, stream>>>(                           \
      d.codes, d.scales, d.global_dec, nparts, gpr, d.ld_y, d.y)
  if (d.out_f32) { if (d.blocking) NVFP4_DQ(true, true); else NVFP4_DQ(true, false); }
  else { if (d.blocking) NVFP4_DQ(false, true); else NVFP4_DQ(false, false); }
#undef NVFP4_DQ
  return hipGetLastError();
}

}  // namespace nvfp4
