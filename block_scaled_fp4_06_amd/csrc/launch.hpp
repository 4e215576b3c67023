// launch.hpp -- internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Quantization workspace: a block of coordination words, then one 64-bit word per chunk of
// the input (see quantize.hip).  8 MiB covers the largest tensor the ABI accepts.
constexpr size_t kCoordBytes = 8192;
constexpr size_t kWorkspaceBytes = ((size_t)8 << 20) + kCoordBytes;

// Chunks the quantization kernel divides a rows x cols tensor into.
uint64_t quantize_chunks(int64_t rows, int64_t cols, int blocking, int rounding);

struct QuantLaunch {
  const uint16_t *x;
  int64_t rows, cols, ld;
  int blocking;           // 0: 1x16, 1: 16x16
  int rounding;           // 0: nearest-even, 1: stochastic
  int rht;                // 1: RHT-16 along rows
  uint32_t rht_k0, rht_k1; // RHT seed (Philox key of the sign vector)
  uint32_t sr_k0, sr_k1;  // Philox key
  uint64_t sr_base;       // Philox element index of x[0][0]
  uint8_t *codes, *scales;
  float *global_dec;
  uint8_t *codes_t, *scales_t;
  uint32_t *dev_status;
  void *ws;               // workspace (kCoordBytes + 8 bytes per chunk), zero-filled once
};

hipError_t launch_quantize(const QuantLaunch &q, hipStream_t stream);


struct DequantLaunch {
  const uint8_t *codes, *scales;
  const float *global_dec;
  int64_t rows, cols, ld_y;
  int blocking;
  int out_f32;
  void *y;
};

hipError_t launch_dequantize(const DequantLaunch &d, hipStream_t stream);

struct GemmOperand {
  const uint8_t *codes, *scales;
  const float *global_dec;
  int blocking;
};

struct GemmLaunch {
  GemmOperand a, b;
  int64_t M, N, K, ldc;
  int out_f32;
  void *c;
  void *ws = nullptr;   // optional: lets the last, partial round of tiles split along K
};

// GEMM workspace: one arrival counter per split tile, then the fp32 partial tiles (256 x
// 256) of at most kGemmMaxItems split work items.
constexpr size_t kGemmCtrBytes = 4096;
constexpr int kGemmMaxItems = 256;
constexpr size_t kGemmWorkspaceBytes = kGemmCtrBytes + (size_t)kGemmMaxItems * 256 * 256 * 4;

hipError_t launch_gemm(const GemmLaunch &g, hipStream_t stream);

// MXFP4 (mxfp4.hip): 32-element blocks, one E8M0 scale byte each, no tensor scale.
struct MxQuantLaunch {
  const uint16_t *x;
  int64_t rows, cols, ld;
  uint8_t *codes, *scales;
};

hipError_t launch_mx_quantize(const MxQuantLaunch &q, hipStream_t stream);

struct MxDequantLaunch {
  const uint8_t *codes, *scales;
  int64_t rows, cols, ld_y;
  int out_f32;
  void *y;
};

hipError_t launch_mx_dequantize(const MxDequantLaunch &d, hipStream_t stream);

struct MxGemmLaunch {
  const uint8_t *a_codes, *a_scales, *b_codes, *b_scales;
  int64_t M, N, K, ldc;
  int out_f32;
  void *c;
};

hipError_t launch_mx_gemm(const MxGemmLaunch &g, hipStream_t stream);

struct TransposeLaunch {
  const uint16_t *x;
  int64_t rows, cols, ld_x;
  uint16_t *y;
  int64_t ld_y;
};

hipError_t launch_transpose_bf16(const TransposeLaunch &t, hipStream_t stream);

}  // namespace nvfp4
