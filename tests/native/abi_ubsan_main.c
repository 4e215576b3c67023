// abi_ubsan_main.c -- drives every entry point of the C ABI with extreme arguments
// (test only).  Built host-only with UndefinedBehaviorSanitizer (halting on the first
// report) together with api.hip and launch_stubs.hip, so that no kernel is launched: an
// argument error must come back with its status, and a call that passes the checks ends in
// a stub that returns NVFP4_ERR_HIP.  Exit status 0 and the line "abi ubsan ok" mean every
// expectation held and the sanitizer found nothing.
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>

#include "nvfp4.h"

extern int stub_calls;
extern int64_t stub_rows, stub_cols, stub_ld;

static int failures = 0;
static void expect(const char *what, int line, nvfp4_status got, nvfp4_status want) {
  if (got != want) {
    fprintf(stderr, "line %d: %s: status %d, expected %d\n", line, what, (int)got, (int)want);
    ++failures;
  }
}
#define EXPECT(call, want) expect(#call, __LINE__, (call), (want))

// Aligned stand-in addresses; never dereferenced (the stubs launch nothing).
#define X ((uint16_t *)0x10000)
#define B ((uint8_t *)0x20000)
#define G ((float *)0x30000)
#define W ((void *)0x40000)

static nvfp4_status quant(int64_t rows, int64_t cols, int64_t ld, int blocking, int rounding,
                          int rht, int transpose) {
  nvfp4_quant_params p = {blocking, rounding, rht, 0, 1, 2, 0};
  return nvfp4_quantize(X, rows, cols, ld, &p, B, B, G, transpose ? B : NULL,
                        transpose ? B : NULL, NULL, W, nvfp4_quantize_workspace_bytes(), NULL);
}

int main() {
  const int64_t i64max = INT64_MAX, i64min = INT64_MIN;
  // shapes whose element count overflows or wraps a 64-bit product, and the extremes
  const int64_t huge[][2] = {{(int64_t)1 << 34, (int64_t)1 << 34},
                             {(int64_t)1 << 32, (int64_t)1 << 32},
                             {((int64_t)1 << 33) + 16, (int64_t)1 << 31},
                             {((int64_t)1 << 35) + 16, 16},
                             {i64max - 15, 16},
                             {16, i64max - 15},
                             {i64max - 15, i64max - 15}};
  for (size_t h = 0; h < sizeof huge / sizeof huge[0]; ++h) {
    const int64_t r = huge[h][0], c = huge[h][1];
    for (int blk = 0; blk < 2; ++blk)
      for (int rnd = 0; rnd < 2; ++rnd)
        for (int rht = 0; rht < 2; ++rht) {
          EXPECT(quant(r, c, c, blk, rnd, rht, 0), NVFP4_ERR_SHAPE);
          if (blk == 1) EXPECT(quant(r, c, c, blk, rnd, rht, 1), NVFP4_ERR_SHAPE);
        }
    for (int blk = 0; blk < 2; ++blk)
      for (int od = 0; od < 2; ++od)
        EXPECT(nvfp4_dequantize(B, B, G, r, c, blk, W, c, od, NULL), NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_transpose_bf16(X, r, c, c, X, r, NULL), NVFP4_ERR_SHAPE);
    const int64_t mc = c & ~(int64_t)31;
    if (mc) {
      EXPECT(mxfp4_quantize(X, r, mc, mc, B, B, NULL), NVFP4_ERR_SHAPE);
      EXPECT(mxfp4_dequantize(B, B, r, mc, W, mc, 0, NULL), NVFP4_ERR_SHAPE);
    }
    nvfp4_operand op = {B, B, G, 0, 0};
    EXPECT(nvfp4_gemm(&op, &op, r, c, 64, W, c, 0, NULL), NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_gemm(&op, &op, 64, 64, r > c ? r : c, W, 64, 0, NULL), NVFP4_ERR_SHAPE);
    EXPECT(mxfp4_gemm(B, B, B, B, r, c, 64, W, c, 0, NULL), NVFP4_ERR_SHAPE);
  }
  // strides whose span (rows - 1) * ld + cols overflows, negative and extreme arguments
  const int64_t lds[] = {i64max, i64max - 7, (int64_t)1 << 62, i64min, -16};
  for (size_t i = 0; i < sizeof lds / sizeof lds[0]; ++i) {
    const int64_t ld = lds[i];
    EXPECT(quant(32, 32, ld, 0, 0, 1, 0), NVFP4_ERR_SHAPE);
    EXPECT(quant(32, 32, ld, 1, 1, 0, 1), NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_dequantize(B, B, G, 32, 32, 0, W, ld, 1, NULL), NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_transpose_bf16(X, 32, 64, ld, X, 32, NULL), NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_transpose_bf16(X, 32, 64, 64, X, ld, NULL), NVFP4_ERR_SHAPE);
    EXPECT(mxfp4_quantize(X, 32, 64, ld, B, B, NULL), NVFP4_ERR_SHAPE);
    EXPECT(mxfp4_dequantize(B, B, 32, 64, W, ld, 0, NULL), NVFP4_ERR_SHAPE);
    nvfp4_operand op = {B, B, G, 0, 0};
    EXPECT(nvfp4_gemm(&op, &op, 32, 32, 64, W, ld, 0, NULL), NVFP4_ERR_SHAPE);
    EXPECT(mxfp4_gemm(B, B, B, B, 32, 32, 64, W, ld, 0, NULL), NVFP4_ERR_SHAPE);
  }
  const int64_t bad[] = {i64min, i64max, -16, -1};
  for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
    const int64_t v = bad[i];
    EXPECT(quant(v, 32, 32, 0, 0, 0, 0), NVFP4_ERR_SHAPE);
    EXPECT(quant(32, v, 32, 0, 0, 0, 0), NVFP4_ERR_SHAPE);
    nvfp4_operand op = {B, B, G, 0, 0};
    EXPECT(nvfp4_gemm(&op, &op, v, 32, 64, W, 32, 0, NULL), NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_gemm(&op, &op, 32, v, 64, W, 32, 0, NULL), NVFP4_ERR_SHAPE);
    EXPECT(nvfp4_gemm(&op, &op, 32, 32, v, W, 32, 0, NULL), NVFP4_ERR_SHAPE);
    EXPECT(mxfp4_gemm(B, B, B, B, 32, 32, v, W, 32, 0, NULL), NVFP4_ERR_SHAPE);
  }
  if (stub_calls != 0) {
    fprintf(stderr, "%d rejected calls reached a launcher\n", stub_calls);
    ++failures;
  }
  // the largest tensor each call accepts passes the checks and reaches its launcher
  const int64_t n35 = (int64_t)1 << 35;
  for (int blk = 0; blk < 2; ++blk)
    for (int rnd = 0; rnd < 2; ++rnd) {
      stub_calls = 0;
      EXPECT(quant(n35 / 4096, 4096, 4096, blk, rnd, 1, blk == 1), NVFP4_ERR_HIP);
      if (stub_calls != 1 || stub_rows != n35 / 4096 || stub_cols != 4096) ++failures;
    }
  EXPECT(nvfp4_dequantize(B, B, G, n35 / 16, 16, 0, W, 16, 0, NULL), NVFP4_ERR_HIP);
  EXPECT(nvfp4_transpose_bf16(X, n35 / 8, 8, 8, X, n35 / 8, NULL), NVFP4_ERR_HIP);
  EXPECT(mxfp4_quantize(X, n35 / 64, 32, 32, B, B, NULL), NVFP4_ERR_HIP);
  /* a long row stride within the span limit */
  const int64_t ld_max = (((int64_t)1 << 60) - 16) / 15 & ~(int64_t)7;
  EXPECT(quant(16, 16, ld_max, 0, 0, 0, 0), NVFP4_ERR_HIP);
  if (stub_ld != ld_max) ++failures;
  nvfp4_operand op = {B, B, G, 1, 0};
  EXPECT(nvfp4_gemm(&op, &op, (int64_t)1 << 30, 256, (int64_t)1 << 23, W, 256, 0, NULL),
         NVFP4_ERR_HIP);
  /* a C caller may pass any int as the status */
  for (int s = -1; s < 100; ++s)
    if (!nvfp4_status_string((nvfp4_status)s)) ++failures;
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("abi ubsan ok\n");
  return 0;
}
