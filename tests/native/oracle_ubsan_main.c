/*
 * oracle_ubsan_main.c -- runs the CPU oracle (oracle/nvfp4_oracle.c) under
 * UndefinedBehaviorSanitizer, halting on the first report (test only).
 *
 * Every entry point is driven with small tensors holding the edge values of the formats
 * (zeros of both signs, bf16 subnormals, the largest finite bf16, values at the E2M1
 * decision points, inf and NaN), with both blockings, both roundings and the transform,
 * and the scalar codecs with every E4M3 and E2M1 code and a sweep of binary32 patterns.
 * Exit status 0 and "oracle ubsan ok" mean the sanitizer found nothing and the few
 * structural expectations below held.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "nvfp4_oracle.h"

static int failures = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "line %d: %s\n", __LINE__, #c);             \
            ++failures;                                                 \
        }                                                               \
    } while (0)

static uint16_t f32_bits_to_bf16_trunc(uint32_t u) { return (uint16_t)(u >> 16); }

/* A rows x cols bf16 tensor: a deterministic mix of ordinary values and edge values. */
static void fill(uint16_t *x, int64_t rows, int64_t cols, int64_t ld, uint32_t seed,
                 int with_nonfinite)
{
    const int64_t n = rows * ld;
    static const uint16_t edge[] = {
        0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F, /* 0, -0, subnormals, max */
        0x3E80, 0x3F40, 0x3FA0, 0x3FE0, 0x4020, 0x4060, 0x40A0, 0x40C0, /* E2M1 decision points */
        0x3F80, 0xBF80, 0x4440, 0xC440};
    uint32_t s = seed * 2654435761u + 1u;
    for (int64_t i = 0; i < n; ++i) {
        s = s * 1664525u + 1013904223u;
        if ((s >> 28) == 0) {
            x[i] = edge[(s >> 8) % (sizeof edge / sizeof edge[0])];
        } else {
            /* finite values over a wide exponent range */
            const uint32_t e = 100u + ((s >> 8) % 60u);
            x[i] = f32_bits_to_bf16_trunc(((s & 0x80000000u)) | (e << 23) | ((s >> 4) & 0x7FFFFFu));
        }
    }
    if (with_nonfinite) {
        x[1] = 0x7F80;                          /* inf */
        x[(rows - 1) * ld + cols - 2] = 0x7FC1; /* NaN */
    }
}

static void run_quantize(int64_t rows, int64_t cols, int64_t ld, uint32_t seed)
{
    uint16_t *x = calloc((size_t)(rows * ld + 16), sizeof *x);
    uint8_t *codes = calloc((size_t)(rows * cols / 2 + 16), 1);
    uint8_t *scales = calloc((size_t)(rows * cols / 16 + 16), 1);
    float *y = calloc((size_t)(rows * cols + 16), sizeof *y);
    double *v = calloc((size_t)(rows * cols + 16), sizeof *v);
    for (int nf = 0; nf < 2; ++nf) {
        fill(x, rows, cols, ld, seed + (uint32_t)nf, nf);
        for (int blk = 0; blk < 2; ++blk)
            for (int rnd = 0; rnd < 2; ++rnd)
                for (int rht = 0; rht < 2; ++rht) {
                    orc_params p = {blk, rnd, rht, 0, 0x5248u + seed, 7u + seed, 16u * seed};
                    float g = 0.0f;
                    uint32_t st = 0;
                    const int rc = orc_quantize(x, rows, cols, ld, &p, codes, scales, &g, &st);
                    /* the transform of the largest bf16 values overflows binary32: then the
                       tensor is non-finite too */
                    CHECK(rc == (int)st && (nf ? rc == 1 : (rht || rc == 0)));
                    CHECK(rc ? isnan(g) : (g > 0.0f && isfinite(g)));
                    if (!rc) {
                        CHECK(orc_dequantize(codes, scales, g, rows, cols, blk, y) == 0);
                        CHECK(orc_block_values_f64(codes, scales, rows, cols, blk, v) == 0);
                    }
                }
    }
    if (cols % 32 == 0) {
        uint32_t st = 0;
        CHECK(orc_mx_quantize(x, rows, cols, ld, codes, scales, &st) == 1);
        CHECK(orc_mx_block_values_f64(codes, scales, rows, cols, v) == 0);
    }
    free(x);
    free(codes);
    free(scales);
    free(y);
    free(v);
}

int main(void)
{
    /* tensors: ragged against the 16x16 tiles, strided, one row, all zeros */
    run_quantize(16, 16, 16, 1);
    run_quantize(48, 96, 104, 2);
    run_quantize(32, 160, 160, 3);
    {
        uint16_t z[16 * 32] = {0};
        uint8_t c[16 * 16], s[32];
        float g = 0.0f, y[16 * 32];
        uint32_t st = 1;
        orc_params p = {0, 0, 1, 0, 1, 2, 0};
        CHECK(orc_quantize(z, 16, 32, 32, &p, c, s, &g, &st) == 0 && g == 1.0f && st == 0);
        CHECK(orc_dequantize(c, s, g, 16, 32, 0, y) == 0);
        CHECK(orc_quantize(z, 0, 32, 32, &p, c, s, &g, &st) == 0);
    }
    /* rejected shapes */
    {
        orc_params p = {0, 0, 0, 0, 0, 0, 0};
        uint8_t c[256], s[256];
        float g, y[256];
        uint32_t st;
        const int64_t bad[][3] = {{-16, 16, 16}, {16, -16, 16}, {15, 16, 16}, {16, 8, 16},
                                  {16, 16, 8}, {INT64_MIN, 16, 16}, {16, INT64_MIN, 16}};
        for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
            CHECK(orc_quantize(NULL, bad[i][0], bad[i][1], bad[i][2], &p, c, s, &g, &st) == -1);
            CHECK(orc_dequantize(c, s, 1.0f, bad[i][0], bad[i][1], 0, y) == -1 ||
                  bad[i][2] == 8);
        }
        CHECK(orc_mx_quantize(NULL, 16, 48, 48, c, s, &st) == -1);
    }
    /* scalar codecs: every code, and a sweep of binary32 patterns (both signs, inf, NaN) */
    for (int c = 0; c < 256; ++c) {
        const float d = orc_e4m3_decode((uint8_t)c);
        if (!isnan(d))
            CHECK(orc_e4m3_encode(fabsf(d)) == (uint8_t)(c & 0x7F) || d == 0.0f);
        (void)orc_mx_scale_value((uint8_t)c);
    }
    for (int c = 0; c < 16; ++c)
        CHECK(orc_e2m1_encode_rn(orc_e2m1_decode((uint8_t)c)) == (uint8_t)c);
    for (uint64_t u = 0; u <= 0xFFFFFFFFull; u += 65537u) {
        float f;
        const uint32_t b = (uint32_t)u;
        memcpy(&f, &b, sizeof f);
        (void)orc_f32_to_bf16(f);
        (void)orc_mx_scale(fabsf(f));
        if (!isnan(f)) {
            (void)orc_e4m3_encode(fabsf(f));
            (void)orc_e2m1_encode_rn(f);
            (void)orc_e2m1_encode_sr(f, (uint16_t)(b * 40503u));
        }
    }
    /* the Philox stream and the transform at extreme counters and keys */
    {
        const uint32_t ctr[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
        const uint32_t key[2] = {0xFFFFFFFFu, 0xFFFFFFFFu};
        uint32_t out[4];
        uint16_t k[64];
        float d[16], xv[16], yv[16];
        orc_philox4x32_10(ctr, key, out);
        orc_sr_bits_array(UINT64_MAX, UINT64_MAX - 63u, 64, k);
        orc_rht_signs(UINT64_MAX, d);
        for (int j = 0; j < 16; ++j)
            xv[j] = (j & 1) ? 3.0e38f : -3.0e38f;
        orc_rht16(xv, d, yv);
    }
    CHECK(orc_abi_version() > 0);
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle ubsan ok\n");
    return 0;
}
