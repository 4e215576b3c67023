// launch.hpp -- internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"

namespace nvfp4 {


// Work division of the quantization kernels (quantize.hip), shared with the argument checks.
// 1x16, nearest-even: a chunk is kT1 threads x kG1 row groups of 16 elements.
constexpr int kT1 = 512;
constexpr int kG1 = 20;
constexpr uint32_t kChunk1 = (uint32_t)kT1 * kG1;
// 1x16, stochastic: pass 1 writes one 32-bit partial maximum per workgroup.
constexpr uint32_t kAmaxMaxWg = 1024;
// 16x16: a chunk is up to kG16 tile-rows x 16 tile-columns.
constexpr int kG16 = 8;

// Quantization workspace (see quantize.hip): a header of coordination words, one 64-bit
// word per chunk for the single-read kernels (8 MiB covers the largest tensor the ABI
// accepts: 2^20 chunks of 16x16 blocks), then the pass-1 partial maxima of the two-pass
// stochastic path in a region of their own, so that no word one path writes is ever read
// by the other as its own.
constexpr size_t kCoordBytes = 8192;
constexpr size_t kWordsBytes = (size_t)8 << 20;
constexpr size_t kPartialsOffset = kCoordBytes + kWordsBytes;
constexpr size_t kWorkspaceBytes = kPartialsOffset + 4 * (size_t)kAmaxMaxWg;

// Chunk words the single-read kernels need after the workspace header for a rows x cols
// tensor (rows, cols >= 0, multiples of 16, rows * cols <= 2^35): one per chunk; none for
// the two-pass path (stochastic rounding with 1x16 blocks), whose partials have their own
// region.
inline uint64_t quantize_chunks(int64_t rows, int64_t cols, int blocking, int rounding) {
  if (blocking == 0) {
    if (rounding == 1) return 0;
    return ((uint64_t)rows * (uint64_t)(cols / 16) + kChunk1 - 1) / kChunk1;
  }
  return (((uint64_t)(rows / 16) + kG16 - 1) / kG16) * (((uint64_t)(cols / 16) + 15) / 16);
}

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

// The argument checks of nvfp4_quantize other than its workspace (api.hip); on success
// fills q, with q->ws = nullptr.  Makes no HIP call.
nvfp4_status check_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                            const nvfp4_quant_params *p, uint8_t *codes, uint8_t *scales,
                            float *global_dec, uint8_t *codes_t, uint8_t *scales_t,
                            uint32_t *dev_status, QuantLaunch *q);


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
