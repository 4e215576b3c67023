// api.hip -- the C ABI of libnvfp4 (declared in include/nvfp4.h).
//
// Every argument check happens here, before any HIP call, so a bad call returns its
// status synchronously and can be exercised on a machine without a GPU.  After the
// checks the call only marshals arguments into a launch description; all arithmetic
// runs in the HIP kernels.
#include "nvfp4.h"

#include <string.h>

#include "launch.hpp"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool mult16(int64_t v) { return v >= 0 && (v & 15) == 0; }

// Largest element count handled with 32-bit group indices.
constexpr int64_t kMaxElems = (int64_t)1 << 35;
// MXFP4 kernels index 8-element pieces with 32 bits.
constexpr int64_t kMaxMxElems = (int64_t)1 << 34;
// Largest element offset (r * ld + c) of a strided tensor: far beyond any memory, and small
// enough that the kernels' 64-bit byte addresses (at most 4 bytes per element) never wrap.
constexpr int64_t kMaxSpan = (int64_t)1 << 60;

// rows x cols elements, both >= 0, at most `max` of them.  The bound is checked by division,
// so no product is formed that could overflow.
bool count_ok(int64_t rows, int64_t cols, int64_t max) {
  return rows >= 0 && cols >= 0 && (cols == 0 || rows <= max / cols);
}

// A rows x cols tensor with row stride ld (>= cols >= 0) spans (rows - 1) * ld + cols
// elements; that must stay within kMaxSpan (checked without an overflowing product).
bool span_ok(int64_t rows, int64_t cols, int64_t ld) {
  if (rows <= 1) return cols <= kMaxSpan;
  return ld <= (kMaxSpan - cols) / (rows - 1);
}

// The GEMMs launch one workgroup per 128 x 128 (or larger) tile of C on a one-dimensional
// grid, whose size is a 32-bit signed count.
bool too_many_tiles(int64_t M, int64_t N) {
  return ((M + 127) / 128) * ((N + 127) / 128) > (int64_t)0x7FFFFFFF;
}

nvfp4_status from_hip(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

}  // namespace

extern "C" {

size_t nvfp4_quantize_workspace_bytes(void) { return nvfp4::kWorkspaceBytes; }

}  // extern "C"

namespace nvfp4 {

nvfp4_status check_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                            const nvfp4_quant_params *p, uint8_t *codes, uint8_t *scales,
                            float *global_dec, uint8_t *codes_t, uint8_t *scales_t,
                            uint32_t *dev_status, QuantLaunch *q) {
  if (!p) return NVFP4_ERR_NULL;
  if (!mult16(rows) || !mult16(cols) || ld_x < cols || !count_ok(rows, cols, kMaxElems) ||
      !span_ok(rows, cols, ld_x))
    return NVFP4_ERR_SHAPE;
  if (p->blocking != NVFP4_BLOCK_1x16 && p->blocking != NVFP4_BLOCK_16x16)
    return NVFP4_ERR_UNSUPPORTED;
  if (p->rounding != NVFP4_ROUND_RNE && p->rounding != NVFP4_ROUND_STOCHASTIC)
    return NVFP4_ERR_UNSUPPORTED;
  if ((p->rht != 0 && p->rht != 1) || p->reserved != 0) return NVFP4_ERR_UNSUPPORTED;
  if ((codes_t != nullptr) != (scales_t != nullptr)) return NVFP4_ERR_NULL;
  if (codes_t && p->blocking != NVFP4_BLOCK_16x16) return NVFP4_ERR_UNSUPPORTED;
  if (p->rounding == NVFP4_ROUND_STOCHASTIC && (p->sr_index_base & 15u)) return NVFP4_ERR_SHAPE;
  const bool empty = rows == 0 || cols == 0;  // data pointers of empty tensors may be NULL
  if (!global_dec || (!empty && (!x || !codes || !scales))) return NVFP4_ERR_NULL;
  if ((ld_x & 7) || !aligned16(x) || !aligned16(codes) || !aligned16(scales) ||
      !aligned16(global_dec) || (codes_t && !aligned16(codes_t)) ||
      (scales_t && !aligned16(scales_t)) || (dev_status && !aligned16(dev_status)))
    return NVFP4_ERR_ALIGN;
  q->x = x;
  q->rows = rows;
  q->cols = cols;
  q->ld = ld_x;
  q->blocking = p->blocking;
  q->rounding = p->rounding;
  q->rht = p->rht;
  q->rht_k0 = (uint32_t)p->rht_seed;
  q->rht_k1 = (uint32_t)(p->rht_seed >> 32);
  q->sr_k0 = (uint32_t)p->sr_seed;
  q->sr_k1 = (uint32_t)(p->sr_seed >> 32);
  q->sr_base = p->sr_index_base;
  q->codes = codes;
  q->scales = scales;
  q->global_dec = global_dec;
  q->codes_t = codes_t;
  q->scales_t = scales_t;
  q->dev_status = dev_status;
  q->ws = nullptr;
  return NVFP4_OK;
}

}  // namespace nvfp4

extern "C" {

nvfp4_status nvfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                            const nvfp4_quant_params *p, uint8_t *codes, uint8_t *scales,
                            float *global_dec, uint8_t *codes_t, uint8_t *scales_t,
                            uint32_t *dev_status, void *workspace, size_t workspace_bytes,
                            nvfp4_stream_t stream) {
  nvfp4::QuantLaunch q;
  const nvfp4_status st = nvfp4::check_quantize(x, rows, cols, ld_x, p, codes, scales,
                                                global_dec, codes_t, scales_t, dev_status, &q);
  if (st != NVFP4_OK) return st;
  if (!workspace || workspace_bytes < nvfp4::kWorkspaceBytes) return NVFP4_ERR_WORKSPACE;
  if (nvfp4::kCoordBytes + 8 * nvfp4::quantize_chunks(rows, cols, p->blocking, p->rounding) >
      nvfp4::kPartialsOffset)   // (never for an accepted shape)
    return NVFP4_ERR_WORKSPACE;
  if (!aligned16(workspace)) return NVFP4_ERR_ALIGN;
  q.ws = workspace;
  return from_hip(nvfp4::launch_quantize(q, reinterpret_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales,
                              const float *global_dec, int64_t rows, int64_t cols,
                              int32_t blocking, void *y, int64_t ld_y, int32_t out_dtype,
                              nvfp4_stream_t stream) {
  if (!mult16(rows) || !mult16(cols) || ld_y < cols || !count_ok(rows, cols, kMaxElems) ||
      !span_ok(rows, cols, ld_y))
    return NVFP4_ERR_SHAPE;
  if (blocking != NVFP4_BLOCK_1x16 && blocking != NVFP4_BLOCK_16x16) return NVFP4_ERR_UNSUPPORTED;
  if (out_dtype != NVFP4_OUT_BF16 && out_dtype != NVFP4_OUT_FP32) return NVFP4_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return NVFP4_OK;  // nothing to write
  if (!codes || !scales || !global_dec || !y) return NVFP4_ERR_NULL;
  if ((ld_y & 7) || !aligned16(codes) || !aligned16(scales) || !aligned16(global_dec) ||
      !aligned16(y))
    return NVFP4_ERR_ALIGN;
  nvfp4::DequantLaunch d;
  d.codes = codes;
  d.scales = scales;
  d.global_dec = global_dec;
  d.rows = rows;
  d.cols = cols;
  d.ld_y = ld_y;
  d.blocking = blocking;
  d.out_f32 = out_dtype == NVFP4_OUT_FP32;
  d.y = y;
  return from_hip(nvfp4::launch_dequantize(d, reinterpret_cast<hipStream_t>(stream)));
}

static nvfp4_status gemm_call(const nvfp4_operand *a, const nvfp4_operand *b, int64_t M, int64_t N,
                              int64_t K, void *c, int64_t ldc, int32_t out_dtype, void *ws,
                              nvfp4_stream_t stream) {
  if (!a || !b) return NVFP4_ERR_NULL;
  if (!mult16(M) || !mult16(N) || !mult16(K) || ldc < N || M > (1 << 30) || N > (1 << 30) ||
      K > (1 << 23) || too_many_tiles(M, N) || !span_ok(M, N, ldc))
    return NVFP4_ERR_SHAPE;
  if ((a->blocking != NVFP4_BLOCK_1x16 && a->blocking != NVFP4_BLOCK_16x16) ||
      (b->blocking != NVFP4_BLOCK_1x16 && b->blocking != NVFP4_BLOCK_16x16) || a->reserved ||
      b->reserved)
    return NVFP4_ERR_UNSUPPORTED;
  if (out_dtype != NVFP4_OUT_BF16 && out_dtype != NVFP4_OUT_FP32) return NVFP4_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return NVFP4_OK;  // empty output
  // with K == 0 the operands hold no data (C = 0) but the tensor scales are still read
  if (!a->global_dec || !b->global_dec || !c ||
      (K > 0 && (!a->codes || !a->scales || !b->codes || !b->scales)))
    return NVFP4_ERR_NULL;
  if ((ldc & 7) || !aligned16(a->codes) || !aligned16(a->scales) || !aligned16(a->global_dec) ||
      !aligned16(b->codes) || !aligned16(b->scales) || !aligned16(b->global_dec) || !aligned16(c))
    return NVFP4_ERR_ALIGN;
  nvfp4::GemmLaunch g;
  g.a = {a->codes, a->scales, a->global_dec, a->blocking};
  g.b = {b->codes, b->scales, b->global_dec, b->blocking};
  g.M = M;
  g.N = N;
  g.K = K;
  g.ldc = ldc;
  g.out_f32 = out_dtype == NVFP4_OUT_FP32;
  g.c = c;
  g.ws = ws;
  return from_hip(nvfp4::launch_gemm(g, reinterpret_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_gemm(const nvfp4_operand *a, const nvfp4_operand *b, int64_t M, int64_t N,
                        int64_t K, void *c, int64_t ldc, int32_t out_dtype,
                        nvfp4_stream_t stream) {
  return gemm_call(a, b, M, N, K, c, ldc, out_dtype, nullptr, stream);
}

size_t nvfp4_gemm_workspace_bytes(void) { return nvfp4::kGemmWorkspaceBytes; }

nvfp4_status nvfp4_gemm_ws(const nvfp4_operand *a, const nvfp4_operand *b, int64_t M, int64_t N,
                           int64_t K, void *c, int64_t ldc, int32_t out_dtype, void *workspace,
                           size_t workspace_bytes, nvfp4_stream_t stream) {
  if (!workspace || workspace_bytes < nvfp4::kGemmWorkspaceBytes) return NVFP4_ERR_WORKSPACE;
  if (!aligned16(workspace)) return NVFP4_ERR_ALIGN;
  return gemm_call(a, b, M, N, K, c, ldc, out_dtype, workspace, stream);
}

nvfp4_status mxfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                            uint8_t *codes, uint8_t *scales, nvfp4_stream_t stream) {
  if (rows < 0 || cols < 0 || (cols & 31) || ld_x < cols || !count_ok(rows, cols, kMaxMxElems) ||
      !span_ok(rows, cols, ld_x))
    return NVFP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return NVFP4_OK;  // nothing to write
  if (!x || !codes || !scales) return NVFP4_ERR_NULL;
  if ((ld_x & 7) || !aligned16(x) || !aligned16(codes) || !aligned16(scales))
    return NVFP4_ERR_ALIGN;
  nvfp4::MxQuantLaunch q;
  q.x = x;
  q.rows = rows;
  q.cols = cols;
  q.ld = ld_x;
  q.codes = codes;
  q.scales = scales;
  return from_hip(nvfp4::launch_mx_quantize(q, reinterpret_cast<hipStream_t>(stream)));
}

nvfp4_status mxfp4_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                              int64_t cols, void *y, int64_t ld_y, int32_t out_dtype,
                              nvfp4_stream_t stream) {
  if (rows < 0 || cols < 0 || (cols & 31) || ld_y < cols || !count_ok(rows, cols, kMaxMxElems) ||
      !span_ok(rows, cols, ld_y))
    return NVFP4_ERR_SHAPE;
  if (out_dtype != NVFP4_OUT_BF16 && out_dtype != NVFP4_OUT_FP32) return NVFP4_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (!codes || !scales || !y) return NVFP4_ERR_NULL;
  if ((ld_y & 7) || !aligned16(codes) || !aligned16(scales) || !aligned16(y))
    return NVFP4_ERR_ALIGN;
  nvfp4::MxDequantLaunch d;
  d.codes = codes;
  d.scales = scales;
  d.rows = rows;
  d.cols = cols;
  d.ld_y = ld_y;
  d.out_f32 = out_dtype == NVFP4_OUT_FP32;
  d.y = y;
  return from_hip(nvfp4::launch_mx_dequantize(d, reinterpret_cast<hipStream_t>(stream)));
}

nvfp4_status mxfp4_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                        const uint8_t *b_scales, int64_t M, int64_t N, int64_t K, void *c,
                        int64_t ldc, int32_t out_dtype, nvfp4_stream_t stream) {
  if (M < 0 || N < 0 || K < 0 || (K & 31) || ldc < N || M > (1 << 24) || N > (1 << 24) ||
      K > (1 << 23) || too_many_tiles(M, N) || !span_ok(M, N, ldc))
    return NVFP4_ERR_SHAPE;
  if (out_dtype != NVFP4_OUT_BF16 && out_dtype != NVFP4_OUT_FP32) return NVFP4_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!c || (K > 0 && (!a_codes || !a_scales || !b_codes || !b_scales))) return NVFP4_ERR_NULL;
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(b_codes) ||
      !aligned16(b_scales) || !aligned16(c))
    return NVFP4_ERR_ALIGN;
  nvfp4::MxGemmLaunch g;
  g.a_codes = a_codes;
  g.a_scales = a_scales;
  g.b_codes = b_codes;
  g.b_scales = b_scales;
  g.M = M;
  g.N = N;
  g.K = K;
  g.ldc = ldc;
  g.out_f32 = out_dtype == NVFP4_OUT_FP32;
  g.c = c;
  return from_hip(nvfp4::launch_mx_gemm(g, reinterpret_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_transpose_bf16(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                                  uint16_t *y, int64_t ld_y, nvfp4_stream_t stream) {
  if (rows < 0 || cols < 0 || (rows & 7) || (cols & 7) || ld_x < cols || ld_y < rows ||
      !count_ok(rows, cols, kMaxElems) || !span_ok(rows, cols, ld_x) || !span_ok(cols, rows, ld_y))
    return NVFP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (!x || !y) return NVFP4_ERR_NULL;
  if ((ld_x & 7) || (ld_y & 7) || !aligned16(x) || !aligned16(y)) return NVFP4_ERR_ALIGN;
  nvfp4::TransposeLaunch t;
  t.x = x;
  t.rows = rows;
  t.cols = cols;
  t.ld_x = ld_x;
  t.y = y;
  t.ld_y = ld_y;
  return from_hip(nvfp4::launch_transpose_bf16(t, reinterpret_cast<hipStream_t>(stream)));
}

const char *nvfp4_status_string(nvfp4_status s) {
  // A C caller may pass any int: read the bits as an int, since loading a value outside
  // the enumeration's range as the enum type is undefined in C++.
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "bad shape: sizes must be multiples of 16 and ld >= cols";
    case NVFP4_ERR_ALIGN: return "pointer not 16-byte aligned or leading dimension not a multiple of 8";
    case NVFP4_ERR_UNSUPPORTED: return "unsupported option combination";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

}  // extern "C"
