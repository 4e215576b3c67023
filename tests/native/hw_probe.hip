// hw_probe.hip -- test-only microbenchmarks of the ceilings the kernels are measured against.
//
// Built by __graft_entry__.build() into tests/native/libhw_probe.so and driven by
// tests/test_gpu_hw_ceilings.py.  None of this is part of libnvfp4.  Each entry point
// allocates what it needs, times `reps` back-to-back launches between two events after
// untimed ones (`warm` of them where the caller chooses: the clocks of this chip settle over
// the first dozen or so GEMM-sized launches), frees everything and returns microseconds per launch (negative on a HIP
// error).
//
//  * hwp_mfma_stream: the fp16 matrix-core instruction stream of the NVFP4 GEMM with its
//    operands held in registers: the 256 x 256 tile per 256-thread workgroup, 128 x 128
//    per wave as 4 x 4 blocks of v_mfma_f32_32x32x16_f16 (256 fp32 accumulators per lane),
//    `substeps` sub-steps of 16 instructions per tile; no loads, no dequantization, no
//    epilogue (one store per lane keeps the result alive).  With 2560 workgroups and 320
//    sub-steps it performs the FLOPs of the 8192 x 20480 x 5120 product.  The operands
//    alternate between two register sets of random values shaped like dequantized NVFP4
//    elements (an E2M1 magnitude times a 3-bit mantissa, random sign), so the multiplier
//    inputs change every instruction as they do in the GEMM; `zero` feeds zeros instead.
//    hwp_mfma_stream_operands runs it on the values of a real product's operands.
//  * hwp_mfma_fp4_stream: the same for the MXFP4 GEMM's scaled FP4 instruction.
//  * hwp_read: a streaming read of `bytes` (16 bytes per lane per load, each wave load
//    covering 1 KiB), rotating over `nbuf` buffers so that the 256 MB Infinity Cache does
//    not hold the input.
//  * hwp_write: a streaming write of `bytes` (16 bytes per lane), with ordinary stores
//    (policy 0), non-temporal stores (1) or stores with the agent-scope cache policy, which
//    write through the L2 (2).
//  * hwp_empty: a kernel that does nothing: the per-launch cost of back-to-back launches.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_device.hpp"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

// An E2M1 magnitude (0, .5, 1, 1.5, 2, 3, 4, 6) times 1 + m/8, random sign.
__device__ __forceinline__ _Float16 operand_value(uint32_t h) {
  const uint32_t c = h & 7u;
  const float e2m1 = c < 4u ? 0.5f * (float)c : (float)(2u << ((c - 4u) >> 1)) * ((c & 1u) ? 1.5f : 1.0f);
  const float v = e2m1 * (1.0f + (float)((h >> 3) & 7u) * 0.125f);
  return (_Float16)((h >> 6) & 1u ? -v : v);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_stream_kernel(float *out, int substeps, uint32_t seed, int zero) {
  half8 a0[4], a1[4], b0[4], b1[4];
  const uint32_t lane_id = blockIdx.x * 256u + threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t k = (lane_id * 4u + (uint32_t)i) * 8u + (uint32_t)e;
      a0[i][e] = zero ? (_Float16)0.0f : operand_value(mix32(seed ^ (k * 4u + 0u)));
      a1[i][e] = zero ? (_Float16)0.0f : operand_value(mix32(seed ^ (k * 4u + 1u)));
      b0[i][e] = zero ? (_Float16)0.0f : operand_value(mix32(seed ^ (k * 4u + 2u)));
      b1[i][e] = zero ? (_Float16)0.0f : operand_value(mix32(seed ^ (k * 4u + 3u)));
    }
  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  for (int t = 0; t < substeps; t += 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[i], b0[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[i], b1[j], acc[i][j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[i][j][r];
  out[lane_id] = s;
}

// The same stream with operand values taken from NVFP4 operands (A: M x K with 1x16
// blocks, B: N x K with 16x16 blocks, K-contiguous codes): each lane holds, exactly
// dequantized to fp16 as the GEMM feeds them (e2m1 times the E4M3 block scale, no tensor
// scale), its MFMA operand elements for K = 0..31 of its tile's rows and columns, the two
// 16-element halves alternating between sub-steps.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_stream_operands_kernel(float *out, int substeps, const uint8_t *ac, const uint8_t *as,
                                 const uint8_t *bc, const uint8_t *bs, int M, int N, int K) {
  const int tiles_n = N / 256;
  const int tm = (int)blockIdx.x / tiles_n, tn = (int)blockIdx.x % tiles_n;
  const int wave = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, l32 = lane & 31;
  const int64_t rowb = K / 2, groups = K / 16;
  half8 a0[4], a1[4], b0[4], b1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t ra = (int64_t)tm * 256 + wm * 128 + i * 32 + l32;
    const int64_t rb = (int64_t)tn * 256 + wn * 128 + i * 32 + l32;
    // K elements 16 s + 8 h .. + 7 of set s: 4 code bytes at 8 s + 4 h, block s
    const uint32_t wa0 = *reinterpret_cast<const uint32_t *>(ac + ra * rowb + 4 * h);
    const uint32_t wa1 = *reinterpret_cast<const uint32_t *>(ac + ra * rowb + 8 + 4 * h);
    const uint32_t wb0 = *reinterpret_cast<const uint32_t *>(bc + rb * rowb + 4 * h);
    const uint32_t wb1 = *reinterpret_cast<const uint32_t *>(bc + rb * rowb + 8 + 4 * h);
    const _Float16 sa0 = (_Float16)nvfp4::e4m3_decode(as[ra * groups + 0]);
    const _Float16 sa1 = (_Float16)nvfp4::e4m3_decode(as[ra * groups + 1]);
    const _Float16 sb0 = (_Float16)nvfp4::e4m3_decode(bs[(rb / 16) * groups + 0]);
    const _Float16 sb1 = (_Float16)nvfp4::e4m3_decode(bs[(rb / 16) * groups + 1]);
    a0[i] = nvfp4::dequant8_f16(wa0, sa0);
    a1[i] = nvfp4::dequant8_f16(wa1, sa1);
    b0[i] = nvfp4::dequant8_f16(wb0, sb0);
    b1[i] = nvfp4::dequant8_f16(wb1, sb1);
  }
  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  for (int t = 0; t < substeps; t += 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[i], b0[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[i], b1[j], acc[i][j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[i][j][r];
  out[blockIdx.x * 256u + threadIdx.x] = s;
}

// The MXFP4 GEMM's instruction stream: v_mfma_scale_f32_32x32x64_f8f6f4 with both operands
// FP4 (E2M1 codes, one E8M0 scale byte per 32 K-elements), the same 4 x 4 blocks of 32 x 32
// per wave, 16 instructions per sub-step of K = 64.  mode 0: random codes and scale bytes
// 124..131; mode 1: zeros (scale byte 127); mode 2: the codes and scales of MXFP4 operands
// (A M x K, B N x K, K-contiguous, scales M x K/32 and N x K/32), K = 0..127 of each lane's
// rows, the two 64-element halves alternating between sub-steps.
typedef int v8i __attribute__((ext_vector_type(8)));
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_fp4_stream_kernel(float *out, int substeps, int mode, uint32_t seed, const uint8_t *ac,
                            const uint8_t *as, const uint8_t *bc, const uint8_t *bs, int N, int K) {
  const int wave = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, l32 = lane & 31;
  const uint32_t lane_id = blockIdx.x * 256u + threadIdx.x;
  v8i a[2][4], b[2][4];
  int sa[2][4], sb[2][4];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v4i ca = {0, 0, 0, 0}, cb = {0, 0, 0, 0};
      int xa = 127, xb = 127;
      if (mode == 0) {
        const uint32_t k = (lane_id * 8u + (uint32_t)(st * 4 + i)) * 8u;
        ca = (v4i){(int)mix32(seed ^ k), (int)mix32(seed ^ (k + 1)), (int)mix32(seed ^ (k + 2)), (int)mix32(seed ^ (k + 3))};
        cb = (v4i){(int)mix32(seed ^ (k + 4)), (int)mix32(seed ^ (k + 5)), (int)mix32(seed ^ (k + 6)), (int)mix32(seed ^ (k + 7))};
        const uint32_t e = mix32(seed ^ ~k);
        xa = 124 + (int)(e & 7u);
        xb = 124 + (int)((e >> 3) & 7u);
      } else if (mode == 2) {
        const int tiles_n = N / 256;
        const int64_t ra = (int64_t)((int)blockIdx.x / tiles_n) * 256 + wm * 128 + i * 32 + l32;
        const int64_t rb = (int64_t)((int)blockIdx.x % tiles_n) * 256 + wn * 128 + i * 32 + l32;
        const int64_t rowb = K / 2, groups = K / 32;
        ca = *reinterpret_cast<const v4i *>(ac + ra * rowb + 32 * st + 16 * h);
        cb = *reinterpret_cast<const v4i *>(bc + rb * rowb + 32 * st + 16 * h);
        xa = as[ra * groups + 2 * st + h];
        xb = bs[rb * groups + 2 * st + h];
      }
      a[st][i] = __builtin_shufflevector(ca, (v4i){0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
      b[st][i] = __builtin_shufflevector(cb, (v4i){0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
      sa[st][i] = xa;
      sb[st][i] = xb;
    }
  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  for (int t = 0; t < substeps; t += 2) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              a[st][i], b[st][j], acc[i][j], 4, 4, 0, sa[st][i], 0, sb[st][j]);
  }
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += acc[i][j][r];
  out[lane_id] = sum;
}

__global__ __launch_bounds__(256) void read_kernel(const uint4 *__restrict__ in, uint32_t n16,
                                                   uint32_t *out) {
  uint32_t acc = 0;
  const uint32_t stride = gridDim.x * 512u;
  for (uint32_t base = blockIdx.x * 512u; base < n16; base += stride) {
    const uint32_t i0 = base + threadIdx.x, i1 = i0 + 256u;
    const uint4 v0 = i0 < n16 ? in[i0] : make_uint4(0u, 0u, 0u, 0u);
    const uint4 v1 = i1 < n16 ? in[i1] : make_uint4(0u, 0u, 0u, 0u);
    acc += v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
  }
  if (acc == 0x12345678u) out[blockIdx.x] = acc;
}

template <int POLICY>
__global__ __launch_bounds__(256) void write_kernel(uint4 *out, uint32_t n16, uint32_t per_wg) {
  const uint32_t b = blockIdx.x * per_wg;
  const uint32_t e = min(b + per_wg, n16);
  for (uint32_t i = b + threadIdx.x; i < e; i += 256u) {
    const v4i w = {(int)i, (int)(i ^ 0x55u), (int)(i * 3u), (int)~i};
    if (POLICY == 0) {
      *reinterpret_cast<v4i *>(out + i) = w;
    } else if (POLICY == 1) {
      __builtin_nontemporal_store(w, reinterpret_cast<v4i *>(out + i));
    } else {
      // buffer store with the agent-scope cache policy bit (sc1), relative to this
      // workgroup's range, which the resource bounds
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc(out + b, 0, (int)((e - b) * 16u), 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)((i - b) * 16u), 0, 16);
    }
  }
}

__global__ void empty_kernel(int *p) {
  if (p) p[threadIdx.x] = 0;
}

// Microseconds per launch of `launch` over `reps` launches after `warm` untimed ones.
template <typename F>
double time_launches(F &&launch, int warm, int reps) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return -1.0;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return -1.0;
  }
  for (int i = 0; i < warm; ++i) launch(i);
  double us = -1.0;
  if (hipEventRecord(e0, nullptr) == hipSuccess) {
    for (int i = 0; i < reps; ++i) launch(i);
    float ms = 0.0f;
    if (hipEventRecord(e1, nullptr) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
        hipEventElapsedTime(&ms, e0, e1) == hipSuccess && hipGetLastError() == hipSuccess)
      us = (double)ms * 1000.0 / reps;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return us;
}

}  // namespace

extern "C" {

double hwp_mfma_stream(int workgroups, int substeps, int zero, int warm, int reps) {
  if (workgroups < 1 || substeps < 2 || warm < 0 || reps < 1) return -1.0;
  float *out = nullptr;
  if (hipMalloc(&out, (size_t)workgroups * 256 * sizeof(float)) != hipSuccess) return -1.0;
  const double us = time_launches([&](int i) {
    mfma_stream_kernel<<<workgroups, 256>>>(out, substeps & ~1, 0x9E3779B9u + (uint32_t)i, zero);
  }, warm, reps);
  const bool ok = hipDeviceSynchronize() == hipSuccess;
  (void)hipFree(out);
  return ok ? us : -1.0;
}

// Device pointers of an NVFP4 product's operands (A M x K, 1x16 scales; B N x K, 16x16
// scales); M and N multiples of 256, K of 32.  One workgroup per 256 x 256 tile.
double hwp_mfma_stream_operands(const uint8_t *ac, const uint8_t *as, const uint8_t *bc,
                                const uint8_t *bs, int M, int N, int K, int substeps, int warm,
                                int reps) {
  if (!ac || !as || !bc || !bs || M < 256 || N < 256 || K < 32 || M % 256 || N % 256 || K % 32 ||
      substeps < 2 || warm < 0 || reps < 1)
    return -1.0;
  const int wgs = (M / 256) * (N / 256);
  float *out = nullptr;
  if (hipMalloc(&out, (size_t)wgs * 256 * sizeof(float)) != hipSuccess) return -1.0;
  const double us = time_launches([&](int) {
    mfma_stream_operands_kernel<<<wgs, 256>>>(out, substeps & ~1, ac, as, bc, bs, M, N, K);
  }, warm, reps);
  const bool ok = hipDeviceSynchronize() == hipSuccess;
  (void)hipFree(out);
  return ok ? us : -1.0;
}

// MXFP4 stream: `workgroups` tiles of 256 x 256, `substeps` sub-steps of K = 64.  mode 2
// reads operands (device pointers; M, N multiples of 256, K of 128): then workgroups must be
// (M / 256) * (N / 256).
double hwp_mfma_fp4_stream(int workgroups, int substeps, int mode, const uint8_t *ac,
                           const uint8_t *as, const uint8_t *bc, const uint8_t *bs, int M, int N,
                           int K, int warm, int reps) {
  if (workgroups < 1 || substeps < 2 || mode < 0 || mode > 2 || warm < 0 || reps < 1) return -1.0;
  if (mode == 2 && (!ac || !as || !bc || !bs || M < 256 || N < 256 || K < 128 || M % 256 ||
                    N % 256 || K % 128 || workgroups != (M / 256) * (N / 256)))
    return -1.0;
  float *out = nullptr;
  if (hipMalloc(&out, (size_t)workgroups * 256 * sizeof(float)) != hipSuccess) return -1.0;
  const double us = time_launches([&](int i) {
    mfma_fp4_stream_kernel<<<workgroups, 256>>>(out, substeps & ~1, mode, 0x85EBCA6Bu + (uint32_t)i,
                                                ac, as, bc, bs, N, K);
  }, warm, reps);
  const bool ok = hipDeviceSynchronize() == hipSuccess;
  (void)hipFree(out);
  return ok ? us : -1.0;
}

double hwp_read(uint64_t bytes, int nbuf, int workgroups, int reps) {
  if (bytes < 16 || bytes > (1ull << 34) || nbuf < 1 || nbuf > 64 || workgroups < 1 || reps < 1)
    return -1.0;
  const uint32_t n16 = (uint32_t)(bytes / 16);
  uint4 *bufs[64] = {};
  uint32_t *sink = nullptr;
  bool ok = hipMalloc(&sink, (size_t)workgroups * sizeof(uint32_t)) == hipSuccess;
  for (int b = 0; ok && b < nbuf; ++b)
    ok = hipMalloc(&bufs[b], (size_t)n16 * 16) == hipSuccess &&
         hipMemset(bufs[b], b + 1, (size_t)n16 * 16) == hipSuccess;
  double us = -1.0;
  if (ok) {
    us = time_launches([&](int i) { read_kernel<<<workgroups, 256>>>(bufs[i % nbuf], n16, sink); },
                       nbuf, reps);
    ok = hipDeviceSynchronize() == hipSuccess;
  }
  for (int b = 0; b < nbuf; ++b)
    if (bufs[b]) (void)hipFree(bufs[b]);
  if (sink) (void)hipFree(sink);
  return ok ? us : -1.0;
}

double hwp_write(uint64_t bytes, int policy, int workgroups, int reps) {
  if (bytes < 16 || bytes > (1ull << 31) || policy < 0 || policy > 2 || workgroups < 1 || reps < 1)
    return -1.0;
  const uint32_t n16 = (uint32_t)(bytes / 16);
  const uint32_t per = (n16 + (uint32_t)workgroups - 1) / (uint32_t)workgroups;
  uint4 *buf = nullptr;
  if (hipMalloc(&buf, (size_t)n16 * 16) != hipSuccess) return -1.0;
  const double us = time_launches([&](int) {
    if (policy == 0) write_kernel<0><<<workgroups, 256>>>(buf, n16, per);
    else if (policy == 1) write_kernel<1><<<workgroups, 256>>>(buf, n16, per);
    else write_kernel<2><<<workgroups, 256>>>(buf, n16, per);
  }, 5, reps);
  const bool ok = hipDeviceSynchronize() == hipSuccess;
  (void)hipFree(buf);
  return ok ? us : -1.0;
}

double hwp_empty(int workgroups, int reps) {
  if (workgroups < 1 || reps < 1) return -1.0;
  const double us = time_launches([&](int) { empty_kernel<<<workgroups, 256>>>(nullptr); }, 5, reps);
  return hipDeviceSynchronize() == hipSuccess ? us : -1.0;
}

}  // extern "C"
