/*
 * nvfp4_oracle.c -- plain, slow CPU oracle for NVFP4 block-scaled FP4 quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker the GPU library is compared
 * against.  Only the test-suite, the package smoke check and the benchmark's CPU
 * baseline may load it.  It shares no code, header, table or constant generator
 * with the HIP library, and it includes nothing from it.
 *
 * Sources (cited by page and section; the pages give words, not formulas):
 *   [NV-blog] developer.nvidia.com zh-cn blog "NVFP4 trains with precision of 16-bit
 *             and speed and efficiency of 4-bit", section "用于预训练的 NVFP4 量化配方"
 *             (five bullets: 16-element micro-blocks; E4M3 scales; Hadamard on GEMM
 *             inputs; selective 2D blocks; stochastic rounding).
 *   [LB]      longbridge.com news 254797217, section "NVFP4 预训练量化方案", items 1-5
 *             (same five techniques).
 *   [PR]      prism.simon-ai.net article 7890:
 *               "MVFP4与MXFP4：通过缩放实现低精度推理" -- value 6 with block scale 100 is 600;
 *               "MVFP4格式的核心架构革新" -- 16-element blocks, E4M3 block scale, FP32
 *                                         tensor scale on top of the block scales;
 *               "训练稳定性与敏感层保护策略" -- 16x16 weight blocks so W and W^T agree;
 *               "应对异常值与舍入误差的技术手段" -- Hadamard keeps the norm; stochastic
 *                                         rounding of 0.3 on a {0,1} grid goes up 30%.
 *   [10100]   10100.com article 120561019, section 二(二): FP4 has only 16 values.
 * Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 * 1, 2, 3", SC'11 (round function, multipliers, Weyl key increments).
 *
 * Where the pages are silent the plainest reading is taken; every such reading is
 * marked READING below and listed with its reason in the design notes.
 *
 * Arithmetic: IEEE binary32 with round-to-nearest-even, no contraction of a*b+c into
 * an FMA (built with -ffp-contract=off), no flush of subnormals, correctly rounded
 * division.  Exact comparisons are done in binary64 where that makes them obviously
 * exact.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "nvfp4_oracle.h"

/* ------------------------------------------------------------------------- */
/* E2M1 element format                                                        */
/* ------------------------------------------------------------------------- */

/* The 8 magnitudes of a 4-bit E2M1 value, indexed by the low 3 bits of the code
 * (2 exponent bits, bias 1, 1 mantissa bit; exponent 0 is subnormal with step 0.5).
 * [10100] sec. 二(二): 16 values in total (8 magnitudes x sign); [PR] "MVFP4与MXFP4":
 * the largest magnitude is 6.  READING: the OCP FP4 bit layout s.e1e0.m. */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

float orc_e2m1_decode(uint8_t code)
{
    double m = E2M1_MAG[code & 7u];
    return (code & 8u) ? (float)(-m) : (float)m;
}

/* Round-to-nearest magnitude code of a >= 0 ("conventional deterministic rounding to
 * the nearest representable value", [NV-blog] bullet 5 / [LB] item 5).  READING: ties
 * go to the even code (the one whose mantissa bit is 0), as IEEE round-to-nearest-even
 * does; a >= 6 gives 6 (saturation, since 6 is the largest value). */
static unsigned e2m1_rn_mag(float a)
{
    if (a >= 6.0f)
        return 7u; /* saturate; also keeps huge a (where a-4 and a-6 round alike) at 6 */
    unsigned best = 0;
    double bd = fabs((double)a - E2M1_MAG[0]);
    for (unsigned c = 1; c < 8; ++c) {
        double d = fabs((double)a - E2M1_MAG[c]);
        if (d < bd || (d == bd && (c & 1u) == 0)) {
            best = c;
            bd = d;
        }
    }
    return best;
}

uint8_t orc_e2m1_encode_rn(float v)
{
    unsigned s = signbit(v) ? 8u : 0u;
    return (uint8_t)(s | e2m1_rn_mag(fabsf(v)));
}

/* Stochastic rounding ([NV-blog] bullet 5: round up or down with a probability given
 * by the value's position between the two representable neighbours; [PR]
 * "应对异常值与舍入误差的技术手段": 0.3 on a {0,1} grid rounds to 1 with probability 30%).
 * READING: the uniform variate is u = (k + 1/2) / 2^16 from a 16-bit random integer k;
 * round up iff u < frac where frac = (a - lo) / (hi - lo).  a >= 6 gives 6. */
uint8_t orc_e2m1_encode_sr(float v, uint16_t k)
{
    unsigned s = signbit(v) ? 8u : 0u;
    double a = fabs((double)v);
    if (a >= 6.0)
        return (uint8_t)(s | 7u);
    unsigned lo = 0;
    for (unsigned c = 1; c < 8; ++c)
        if (E2M1_MAG[c] <= a)
            lo = c;
    double frac = (a - E2M1_MAG[lo]) / (E2M1_MAG[lo + 1] - E2M1_MAG[lo]);
    double u = ((double)k + 0.5) / 65536.0;
    unsigned m = (u < frac) ? lo + 1 : lo;
    return (uint8_t)(s | m);
}

/* ------------------------------------------------------------------------- */
/* E4M3 block-scale format                                                    */
/* ------------------------------------------------------------------------- */

/* [NV-blog] bullet 2, [LB] item 2, [PR] "MVFP4格式的核心架构革新": the block scale is an FP8
 * value with 4 exponent and 3 mantissa bits.  READING: OCP E4M3FN -- bias 7, exponent
 * field 0 is subnormal (m * 2^-9), largest finite 448 (code 0x7E), 0x7F is NaN, no
 * infinities.  Block scales are never negative, so only codes 0x00..0x7E occur. */
float orc_e4m3_decode(uint8_t b)
{
    unsigned e = (b >> 3) & 15u, m = b & 7u;
    if ((b & 0x7Fu) == 0x7Fu)
        return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(8.0 + (double)m, (int)e - 10);
    return (float)((b & 0x80u) ? -mag : mag);
}

/* READING: encode = round to nearest representable E4M3 value, ties to the even code,
 * saturating to 448 for anything larger (including +inf).  Input s >= 0.  Written as
 * the definition: search the sorted table of the 127 non-negative finite values. */
static double E4M3_TAB[127]; /* decoded values of codes 0..126, ascending */

__attribute__((constructor)) static void e4m3_table_init(void)
{
    for (int c = 0; c < 127; ++c)
        E4M3_TAB[c] = (double)orc_e4m3_decode((uint8_t)c);
}

uint8_t orc_e4m3_encode(float s)
{
    const double *tab = E4M3_TAB;
    double x = (double)s;
    if (!(x >= 0.0))
        return 0;           /* never reached for finite non-negative input */
    if (x >= tab[126])
        return 126;
    int lo = 0, hi = 126;   /* invariant: tab[lo] <= x < tab[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (tab[mid] <= x)
            lo = mid;
        else
            hi = mid;
    }
    double dlo = x - tab[lo], dhi = tab[hi] - x;
    if (dlo < dhi)
        return (uint8_t)lo;
    if (dhi < dlo)
        return (uint8_t)hi;
    return (uint8_t)((lo & 1) ? hi : lo);
}

/* ------------------------------------------------------------------------- */
/* Philox4x32-10 (SC'11)                                                      */
/* ------------------------------------------------------------------------- */

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u /* golden ratio */
#define PHILOX_W1 0xBB67AE85u /* sqrt(3) - 1 */

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += PHILOX_W0;
            k1 += PHILOX_W1;
        }
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* ------------------------------------------------------------------------- */
/* 16-point random Hadamard transform                                         */
/* ------------------------------------------------------------------------- */

/* READING: the sign vector is bit j (LSB first) of word 0 of Philox4x32-10 with
 * key = (lo32(seed), hi32(seed)) and counter (0, 0, 1, 0); bit 1 means -1. */
void orc_rht_signs(uint64_t seed, float d[16])
{
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t ctr[4] = {0u, 0u, 1u, 0u};
    uint32_t w[4];
    orc_philox4x32_10(ctr, key, w);
    for (int j = 0; j < 16; ++j)
        d[j] = ((w[0] >> j) & 1u) ? -1.0f : 1.0f;
}

/* [NV-blog] bullet 3 / [LB] item 3: a Hadamard transform on GEMM inputs; [PR]
 * "应对异常值与舍入误差的技术手段": a *random* Hadamard transform that keeps the vector's
 * norm.  READING: y = (1/4) * H16 * diag(d) * x with H16 the Sylvester Hadamard matrix,
 * evaluated in binary32 in this fixed order: t = d*x (exact), then butterfly stages
 * h = 1, 2, 4, 8, each replacing (t[i], t[i+h]) by (t[i] + t[i+h], t[i] - t[i+h]) for
 * every i with (i & h) == 0, then y = t * 0.25 (exact unless it underflows). */
void orc_rht16(const float x[16], const float d[16], float y[16])
{
    float t[16];
    for (int i = 0; i < 16; ++i)
        t[i] = d[i] * x[i];
    for (int h = 1; h < 16; h <<= 1) {
        for (int i = 0; i < 16; ++i) {
            if (i & h)
                continue;
            float a = t[i], b = t[i + h];
            t[i] = a + b;
            t[i + h] = a - b;
        }
    }
    for (int i = 0; i < 16; ++i)
        y[i] = t[i] * 0.25f;
}

/* ------------------------------------------------------------------------- */
/* Quantize / dequantize                                                      */
/* ------------------------------------------------------------------------- */

static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t f32_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

/* The 16 transformed values of row r, columns c0..c0+15 (RHT applied when rht != 0). */
static void load_group(const uint16_t *x, int64_t ld, int64_t r, int64_t c0, int rht,
                       const float d[16], float y[16])
{
    float v[16];
    for (int j = 0; j < 16; ++j)
        v[j] = bf16_to_f32(x[r * ld + c0 + j]);
    if (rht)
        orc_rht16(v, d, y);
    else
        for (int j = 0; j < 16; ++j)
            y[j] = v[j];
}

/* The 16-bit random integer of element index i: Philox4x32-10 with
 * key = (lo32(seed), hi32(seed)), counter = (lo32(i >> 3), hi32(i >> 3), 0, 0) gives
 * 128 bits; element i takes bits [16*(i & 7), 16*(i & 7) + 16).  READING. */
static uint16_t sr_bits(uint64_t seed, uint64_t i)
{
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint64_t g = i >> 3;
    uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), 0u, 0u};
    uint32_t w[4];
    orc_philox4x32_10(ctr, key, w);
    unsigned lane = (unsigned)(i & 7u);
    return (uint16_t)(w[lane >> 1] >> (16u * (lane & 1u)));
}

int orc_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                 const orc_params *p, uint8_t *codes, uint8_t *scales, float *global_dec,
                 uint32_t *status)
{
    if (rows < 0 || cols < 0 || rows % 16 || cols % 16 || ld_x < cols)
        return -1;
    if (p->rounding == ORC_ROUND_SR && (p->sr_index_base % 16))
        return -1;

    float d[16];
    orc_rht_signs(p->rht_seed, d);

    /* Step 1: tensor amax over the transformed values.  [PR] "MVFP4格式的核心架构革新":
     * an FP32 per-tensor scale sits on top of the E4M3 block scales and covers the
     * large range.  READING: s_enc = 6*448 / amax maps the tensor's largest magnitude to
     * the top of both formats; the stored (decode) scale is amax / (6*448). */
    float amax = 0.0f;
    int nonfinite = 0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c0 = 0; c0 < cols; c0 += 16) {
            float y[16];
            load_group(x, ld_x, r, c0, p->rht, d, y);
            for (int j = 0; j < 16; ++j) {
                float a = fabsf(y[j]);
                if (!isfinite(a))
                    nonfinite = 1;
                else if (a > amax)
                    amax = a;
            }
        }
    if (status)
        *status = nonfinite ? 1u : 0u;
    if (nonfinite) {
        *global_dec = NAN;
        return 1;
    }
    float s_enc, s_dec;
    if (amax == 0.0f) {
        s_enc = 1.0f;
        s_dec = 1.0f;
    } else {
        s_enc = 2688.0f / amax;
        if (s_enc > FLT_MAX)
            s_enc = FLT_MAX;
        s_dec = amax / 2688.0f;
    }
    *global_dec = s_dec;

    int64_t bh = (p->blocking == ORC_BLOCK_16x16) ? 16 : 1; /* block height */
    int64_t nbr = rows / bh, nbc = cols / 16;

#pragma omp parallel for schedule(static)
    for (int64_t br = 0; br < nbr; ++br) {
        float y[16][16];
        for (int64_t bc = 0; bc < nbc; ++bc) {
            /* Step 2: block amax over the block's 16 (1x16) or 256 (16x16) values.
             * [NV-blog] bullet 1: 16 elements share one scale; [PR]
             * "训练稳定性与敏感层保护策略": weights use 16x16 blocks, 256 values per scale. */
            float bmax = 0.0f;
            for (int64_t i = 0; i < bh; ++i) {
                load_group(x, ld_x, br * bh + i, bc * 16, p->rht, d, y[i]);
                for (int j = 0; j < 16; ++j)
                    if (fabsf(y[i][j]) > bmax)
                        bmax = fabsf(y[i][j]);
            }
            /* Step 3: E4M3 block scale.  READING: sb = e4m3((bmax / 6) * s_enc) in that
             * operation order; its decoded value sbd is what the elements divide by. */
            float sb32 = (bmax / 6.0f) * s_enc;
            uint8_t sb = orc_e4m3_encode(sb32);
            float sbd = orc_e4m3_decode(sb);
            scales[br * nbc + bc] = sb;
            /* Step 4: per-element scale r = s_enc / sbd (0 for a zero scale). */
            float rr;
            if (sbd == 0.0f) {
                rr = 0.0f;
            } else {
                rr = s_enc / sbd;
                if (rr > FLT_MAX)
                    rr = FLT_MAX;
            }
            for (int64_t i = 0; i < bh; ++i) {
                int64_t r = br * bh + i;
                for (int j = 0; j < 16; ++j) {
                    int64_t c = bc * 16 + j;
                    float v = y[i][j] * rr;
                    uint8_t q;
                    if (p->rounding == ORC_ROUND_SR) {
                        uint64_t idx = p->sr_index_base + (uint64_t)r * (uint64_t)cols + (uint64_t)c;
                        q = orc_e2m1_encode_sr(v, sr_bits(p->sr_seed, idx));
                    } else {
                        q = orc_e2m1_encode_rn(v);
                    }
                    /* READING: the code keeps the sign bit of the transformed value, so a
                     * negative value that rounds to zero is stored as -0 (code 8). */
                    q = (uint8_t)((q & 7u) | (signbit(y[i][j]) ? 8u : 0u));
                    uint8_t *dst = &codes[r * (cols / 2) + c / 2];
                    /* READING: even column in the low nibble, odd column in the high nibble. */
                    if (c & 1)
                        *dst = (uint8_t)((*dst & 0x0Fu) | (q << 4));
                    else
                        *dst = (uint8_t)((*dst & 0xF0u) | q);
                }
            }
        }
    }
    return 0;
}

/* [PR] "MVFP4与MXFP4": a stored 4-bit value times its block scale gives the real value
 * (6 with scale 100 stands for 600); with the tensor scale on top
 * ([PR] "MVFP4格式的核心架构革新"): xhat = (e2m1(q) * sbd) * s_dec, the first product exact. */
int orc_dequantize(const uint8_t *codes, const uint8_t *scales, float global_dec,
                   int64_t rows, int64_t cols, int blocking, float *y)
{
    if (rows < 0 || cols < 0 || rows % 16 || cols % 16)
        return -1;
    int64_t bh = (blocking == ORC_BLOCK_16x16) ? 16 : 1;
    int64_t nbc = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t byte = codes[r * (cols / 2) + c / 2];
            uint8_t q = (c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15u);
            float sbd = orc_e4m3_decode(scales[(r / bh) * nbc + c / 16]);
            float e = orc_e2m1_decode(q) * sbd;
            y[r * cols + c] = e * global_dec;
        }
    return 0;
}

/* The same values as orc_dequantize, each rounded to bfloat16 by orc_f32_to_bf16 (nearest,
 * ties to even).  READING: the pages name no output precision of the dequantized tensor;
 * bf16 output rounds the binary32 value once, the usual conversion of that format. */
int orc_dequantize_bf16(const uint8_t *codes, const uint8_t *scales, float global_dec,
                        int64_t rows, int64_t cols, int blocking, uint16_t *y)
{
    if (rows < 0 || cols < 0 || rows % 16 || cols % 16)
        return -1;
    int64_t bh = (blocking == ORC_BLOCK_16x16) ? 16 : 1;
    int64_t nbc = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t byte = codes[r * (cols / 2) + c / 2];
            uint8_t q = (c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15u);
            float sbd = orc_e4m3_decode(scales[(r / bh) * nbc + c / 16]);
            float e = orc_e2m1_decode(q) * sbd;
            y[r * cols + c] = orc_f32_to_bf16(e * global_dec);
        }
    return 0;
}

/* Exact block-scaled values e2m1(q) * sbd (no tensor scale), in binary64: the GEMM
 * reference multiplies these and applies both tensor scales afterwards. */
int orc_block_values_f64(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                         int64_t cols, int blocking, double *out)
{
    if (rows < 0 || cols < 0 || rows % 16 || cols % 16)
        return -1;
    int64_t bh = (blocking == ORC_BLOCK_16x16) ? 16 : 1;
    int64_t nbc = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t byte = codes[r * (cols / 2) + c / 2];
            uint8_t q = (c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15u);
            out[r * cols + c] = (double)orc_e2m1_decode(q) *
                                (double)orc_e4m3_decode(scales[(r / bh) * nbc + c / 16]);
        }
    return 0;
}

/* binary32 -> bfloat16, round to nearest even (NaN stays NaN). */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u = f32_bits(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* ------------------------------------------------------------------------- */
/* Array helpers for the tests                                                */
/* ------------------------------------------------------------------------- */

void orc_f32_to_bf16_array(const float *f, int64_t n, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f32_to_bf16(f[i]);
}

void orc_e4m3_encode_array(const float *s, int64_t n, uint8_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e4m3_encode(s[i]);
}

/* ------------------------------------------------------------------------- */
/* MXFP4: the 32-element, power-of-two-scale format the pages compare NVFP4 with  */
/* ------------------------------------------------------------------------- */
/* [PR] "MVFP4与MXFP4：通过缩放实现低精度推理" and [10100] section 二(一): MXFP4 keeps FP4 E2M1
 * elements with one shared power-of-two (E8M0) scale per 32 elements; NVFP4 uses 16
 * elements and an E4M3 scale.  The pages give no scale rule; READING: the OCP Microscaling
 * Formats specification v1.0 (section 6.3): X = 2^(floor(log2(amax)) - emax) with emax = 2
 * for E2M1 (largest value 6 = 1.5 * 2^2), the exponent clamped to the E8M0 range
 * [-127, 127]; each element is v / X rounded to the nearest E2M1 value (ties to even),
 * saturating at +-6.  A block holding inf or NaN gets the NaN scale 0xFF and zero codes.
 * An all-zero block gets the smallest scale, 2^-127. */
uint8_t orc_mx_scale(float amax)
{
    if (!(amax > 0.0f))
        return 0;                       /* zero block: 2^-127 */
    int e;
    frexpf(amax, &e);                   /* amax = f * 2^e, f in [0.5, 1) */
    int k = (e - 1) - 2;                /* floor(log2(amax)) - emax */
    if (k < -127)
        k = -127;
    if (k > 127)
        k = 127;
    return (uint8_t)(k + 127);
}

double orc_mx_scale_value(uint8_t s)
{
    return s == 0xFF ? NAN : ldexp(1.0, (int)s - 127);
}

/* codes: rows x cols/2 (element 2j in the low nibble), scales: rows x cols/32.  Returns
 * 0, 1 if any block held inf/NaN, -1 for a bad shape (cols % 32 != 0). */
int orc_mx_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                    uint8_t *codes, uint8_t *scales, uint32_t *status)
{
    if (rows < 0 || cols < 0 || cols % 32 || ld_x < cols)
        return -1;
    int nonfinite = 0;
    const int64_t nb = cols / 32;
#pragma omp parallel for schedule(static) reduction(| : nonfinite)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            float v[32];
            float amax = 0.0f;
            int bad = 0;
            for (int j = 0; j < 32; ++j) {
                v[j] = bf16_to_f32(x[r * ld_x + b * 32 + j]);
                if (!isfinite(v[j]))
                    bad = 1;
                else if (fabsf(v[j]) > amax)
                    amax = fabsf(v[j]);
            }
            uint8_t *cp = codes + r * (cols / 2) + b * 16;
            if (bad) {
                nonfinite = 1;
                scales[r * nb + b] = 0xFF;
                for (int j = 0; j < 16; ++j)
                    cp[j] = 0;
                continue;
            }
            const uint8_t s = orc_mx_scale(amax);
            scales[r * nb + b] = s;
            const int k = (int)s - 127;
            for (int j = 0; j < 32; j += 2) {
                /* v / X is a power-of-two scaling: exact unless it lands below the
                 * binary32 normal range, where the value rounds to code 0 either way */
                const uint8_t lo = orc_e2m1_encode_rn(ldexpf(v[j], -k));
                const uint8_t hi = orc_e2m1_encode_rn(ldexpf(v[j + 1], -k));
                cp[j / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    if (status)
        *status = nonfinite ? 1u : 0u;
    return nonfinite ? 1 : 0;
}

/* Exact element values e2m1(q) * X in binary64 (NaN for a NaN scale). */
int orc_mx_block_values_f64(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                            int64_t cols, double *out)
{
    if (rows < 0 || cols < 0 || cols % 32)
        return -1;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            const uint8_t byte = codes[r * (cols / 2) + c / 2];
            const uint8_t q = (c & 1) ? (byte >> 4) : (byte & 0xF);
            out[r * cols + c] = (double)orc_e2m1_decode(q) *
                                orc_mx_scale_value(scales[r * (cols / 32) + c / 32]);
        }
    return 0;
}

void orc_e2m1_encode_rn_array(const float *v, int64_t n, uint8_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e2m1_encode_rn(v[i]);
}

void orc_e2m1_encode_sr_array(const float *v, const uint16_t *k, int64_t n, uint8_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e2m1_encode_sr(v[i], k[i]);
}

void orc_philox_array(const uint32_t *ctr, const uint32_t *key, int64_t n, uint32_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        orc_philox4x32_10(ctr + 4 * i, key + 2 * i, out + 4 * i);
}

void orc_sr_bits_array(uint64_t seed, uint64_t first, int64_t n, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = sr_bits(seed, first + (uint64_t)i);
}

void orc_rht16_rows(const float *x, int64_t ngroups, uint64_t seed, float *y)
{
    float d[16];
    orc_rht_signs(seed, d);
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < ngroups; ++g)
        orc_rht16(x + 16 * g, d, y + 16 * g);
}

void orc_rht16_rows_signs(const float *x, int64_t ngroups, const float d[16], float *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < ngroups; ++g)
        orc_rht16(x + 16 * g, d, y + 16 * g);
}

int orc_abi_version(void) { return 1; }
