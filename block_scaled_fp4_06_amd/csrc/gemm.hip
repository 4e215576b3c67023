// gemm.hip -- NVFP4 x NVFP4 GEMM on gfx950 matrix cores.
//
// C[m][n] = gA * gB * sum_k (e2m1 * e4m3)_A[m][k] * (e2m1 * e4m3)_B[n][k]
// The linear-layer product the recipe exists to accelerate (NVIDIA developer blog zh-cn
// "NVFP4 trains with precision of 16-bit ...", section "用于预训练的 NVFP4 量化配方", the
// Figure 1 paragraph on GEMM throughput).
//
// gfx950's FP4 matrix instructions apply power-of-two (E8M0) scales per 32 K-elements;
// NVFP4 carries an E4M3 scale per 16, whose mantissa cannot be folded into them.  Every
// product e2m1 * e4m3 is exactly representable in fp16 (at most 6 significant bits,
// magnitudes in [2^-10, 2688]), so each tile is dequantized exactly to fp16 in registers
// and fed to v_mfma_f32_32x32x16_f16 with fp32 accumulation; the two tensor scales are
// applied once in the epilogue.
//
// Tiling: 128 x 128 output tile per 256-thread workgroup (2 x 2 waves of 64 x 64, each
// 2 x 2 MFMA blocks of 32 x 32), K step 64.  Packed codes (4 bits per element) and
// scale bytes are staged in LDS; each lane dequantizes its own MFMA operands from LDS.
// Within a 64-wide K step, lane half h (lane / 32) supplies K elements 32h .. 32h+31 in
// four MFMA steps of 8; A and B use the same lane-to-K map, so each MFMA still pairs
// equal k on both sides and the four steps cover the 64 elements once.
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLdsStride = 48;       // LDS bytes per staged row (32 + 16 padding)

struct GemmParams {
  const uint8_t *ac, *as;
  const float *ag;
  const uint8_t *bc, *bs;
  const float *bg;
  int a16, b16;  // 1: 16x16 blocking (scale row = row / 16)
  int M, N, K;
  int64_t ldc;
  void *c;
};

// 16 packed bytes (32 elements) starting at K element kk of a row; `left` = K - kk.
template <bool K32>
__device__ __forceinline__ uint4 load_chunk(const uint8_t *p, int left) {
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (left >= 32) {
    if (K32) {
      v = *reinterpret_cast<const uint4 *>(p);
    } else {
      const uint2 a = reinterpret_cast<const uint2 *>(p)[0];
      const uint2 b = reinterpret_cast<const uint2 *>(p)[1];
      v = make_uint4(a.x, a.y, b.x, b.y);
    }
  } else if (left >= 16) {
    const uint2 a = *reinterpret_cast<const uint2 *>(p);
    v.x = a.x;
    v.y = a.y;
  }
  return v;
}

// Eight E2M1 codes (one dword, element 2i in the low nibble of byte i) times the block
// scale sbd, as eight fp16 values.  Exact: e2m1 * e4m3 fits fp16.
template <bool HWCVT>
__device__ __forceinline__ half8_t dequant8(uint32_t w, _Float16 sbd) {
  half8_t r;
  if (HWCVT) {
    const half2_t s2 = {sbd, sbd};
    const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
    const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
    const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
    const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
    r[0] = p0.x; r[1] = p0.y; r[2] = p1.x; r[3] = p1.y;
    r[4] = p2.x; r[5] = p2.y; r[6] = p3.x; r[7] = p3.y;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t q = (w >> (4 * j)) & 0xFu, m = q & 7u;
      // fp16 bits of the E2M1 magnitude: 0.5 -> 0x3800; m >= 2 -> exponent (m>>1)+14
      const uint32_t mag = m == 0u ? 0u : (m == 1u ? 0x3800u : ((((m >> 1) + 14u) << 10) | ((m & 1u) << 9)));
      const uint16_t bits = (uint16_t)(mag | ((q & 8u) << 12));
      r[j] = __builtin_bit_cast(_Float16, bits) * sbd;
    }
  }
  return r;
}

template <bool F32, bool K32, bool HWCVT>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[kBM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint8_t sB[kBN * kLdsStride];
  __shared__ uint8_t sAs[kBM * 4], sBs[kBN * 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, l32 = lane & 31;
  const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;
  const int64_t rowb = p.K >> 1;
  const int kgroups = p.K >> 4;

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  for (int k0 = 0; k0 < p.K; k0 += kBK) {
    {  // codes: thread -> (row tid/2, 16-byte chunk tid%2)
      const int row = tid >> 1, ch = tid & 1, kk = k0 + 32 * ch;
      uint4 va = make_uint4(0u, 0u, 0u, 0u), vb = va;
      if (m0 + row < p.M) va = load_chunk<K32>(p.ac + (int64_t)(m0 + row) * rowb + (kk >> 1), p.K - kk);
      if (n0 + row < p.N) vb = load_chunk<K32>(p.bc + (int64_t)(n0 + row) * rowb + (kk >> 1), p.K - kk);
      *reinterpret_cast<uint4 *>(sA + row * kLdsStride + 16 * ch) = va;
      *reinterpret_cast<uint4 *>(sB + row * kLdsStride + 16 * ch) = vb;
    }
    {  // scales: threads 0..127 -> A rows, 128..255 -> B rows; 4 K-groups each
      const int row = tid & 127;
      const bool isb = tid >= 128;
      const int grow = (isb ? n0 : m0) + row;
      const bool rv = grow < (isb ? p.N : p.M);
      const uint8_t *sp = isb ? p.bs : p.as;
      const int srow = (isb ? p.b16 : p.a16) ? (grow >> 4) : grow;
      uint8_t *dst = isb ? sBs : sAs;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kg = (k0 >> 4) + j;
        dst[row * 4 + j] = (rv && kg < kgroups) ? sp[(int64_t)srow * kgroups + kg] : (uint8_t)0;
      }
    }
    __syncthreads();

    half8_t aop[2][4], bop[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = wm * 64 + i * 32 + l32;
      const uint4 c = *reinterpret_cast<const uint4 *>(sA + row * kLdsStride + 16 * h);
      const _Float16 s0 = (_Float16)e4m3_decode(sAs[row * 4 + 2 * h]);
      const _Float16 s1 = (_Float16)e4m3_decode(sAs[row * 4 + 2 * h + 1]);
      aop[i][0] = dequant8<HWCVT>(c.x, s0);
      aop[i][1] = dequant8<HWCVT>(c.y, s0);
      aop[i][2] = dequant8<HWCVT>(c.z, s1);
      aop[i][3] = dequant8<HWCVT>(c.w, s1);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = wn * 64 + j * 32 + l32;
      const uint4 c = *reinterpret_cast<const uint4 *>(sB + row * kLdsStride + 16 * h);
      const _Float16 s0 = (_Float16)e4m3_decode(sBs[row * 4 + 2 * h]);
      const _Float16 s1 = (_Float16)e4m3_decode(sBs[row * 4 + 2 * h + 1]);
      bop[j][0] = dequant8<HWCVT>(c.x, s0);
      bop[j][1] = dequant8<HWCVT>(c.y, s0);
      bop[j][2] = dequant8<HWCVT>(c.z, s1);
      bop[j][3] = dequant8<HWCVT>(c.w, s1);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[i][s], bop[j][s], acc[i][j], 0, 0, 0);
    __syncthreads();
  }

  const float alpha = (*p.ag) * (*p.bg);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int col = n0 + wn * 64 + j * 32 + l32;
        if (row < p.M && col < p.N) {
          const float v = acc[i][j][r] * alpha;
          if (F32) {
            reinterpret_cast<float *>(p.c)[(int64_t)row * p.ldc + col] = v;
          } else {
            const uint32_t u = __float_as_uint(v);
            const uint32_t b = ((u & 0x7FFFFFFFu) > 0x7F800000u) ? ((u >> 16) | 0x40u)
                                                                : ((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
            reinterpret_cast<uint16_t *>(p.c)[(int64_t)row * p.ldc + col] = (uint16_t)b;
          }
        }
      }
}

}  // namespace

hipError_t launch_gemm(const GemmLaunch &g, hipStream_t stream) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  GemmParams p;
  p.ac = g.a.codes; p.as = g.a.scales; p.ag = g.a.global_dec; p.a16 = g.a.blocking;
  p.bc = g.b.codes; p.bs = g.b.scales; p.bg = g.b.global_dec; p.b16 = g.b.blocking;
  p.M = (int)g.M; p.N = (int)g.N; p.K = (int)g.K; p.ldc = g.ldc; p.c = g.c;
  const dim3 grid((unsigned)((g.N + kBN - 1) / kBN), (unsigned)((g.M + kBM - 1) / kBM));
  const bool k32 = (g.K % 32) == 0;
#ifndef NVFP4_GEMM_HWCVT
#define NVFP4_GEMM_HWCVT 1
#endif
  constexpr bool hw = NVFP4_GEMM_HWCVT != 0;
  if (g.out_f32) {
    if (k32) gemm_kernel<true, true, hw><<<grid, 256, 0, stream>>>(p);
    else gemm_kernel<true, false, hw><<<grid, 256, 0, stream>>>(p);
  } else {
    if (k32) gemm_kernel<false, true, hw><<<grid, 256, 0, stream>>>(p);
    else gemm_kernel<false, false, hw><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
