/*
 * nvfp4_oracle.h -- C interface of the CPU oracle (test infrastructure only).
 *
 * Host pointers throughout.  Layouts match the GPU library's documented layouts so
 * results compare byte for byte, but nothing here is shared with that library:
 *   codes   rows x cols/2 bytes, row-major, even column in the low nibble;
 *   scales  1x16:  rows x cols/16 bytes; 16x16: rows/16 x cols/16 bytes; row-major;
 *   global  one float, amax / 2688 (1.0 for an all-zero tensor, NaN if non-finite).
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_BLOCK_1x16 = 0, ORC_BLOCK_16x16 = 1 };
enum { ORC_ROUND_RNE = 0, ORC_ROUND_SR = 1 };

typedef struct {
    int32_t blocking;       /* ORC_BLOCK_* */
    int32_t rounding;       /* ORC_ROUND_* */
    int32_t rht;            /* 1: 16-point random Hadamard transform along rows */
    int32_t pad_;
    uint64_t rht_seed;
    uint64_t sr_seed;
    uint64_t sr_index_base; /* element index of x[0][0]; a multiple of 16 */
} orc_params;

float orc_e2m1_decode(uint8_t code);
uint8_t orc_e2m1_encode_rn(float v);
uint8_t orc_e2m1_encode_sr(float v, uint16_t k);
float orc_e4m3_decode(uint8_t b);
uint8_t orc_e4m3_encode(float s);
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
void orc_rht_signs(uint64_t seed, float d[16]);
void orc_rht16(const float x[16], const float d[16], float y[16]);
uint16_t orc_f32_to_bf16(float f);

/* Returns 0 on success, 1 if the input held inf/NaN (global_dec = NaN, *status = 1,
 * codes and scales unspecified), -1 for a bad shape.  With rht the transform runs along
 * each 16-element row group for either blocking (16x16 blocks then cover 16 transformed
 * row groups). */
int orc_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                 const orc_params *p, uint8_t *codes, uint8_t *scales, float *global_dec,
                 uint32_t *status);
int orc_dequantize(const uint8_t *codes, const uint8_t *scales, float global_dec,
                   int64_t rows, int64_t cols, int blocking, float *y);
int orc_dequantize_bf16(const uint8_t *codes, const uint8_t *scales, float global_dec,
                        int64_t rows, int64_t cols, int blocking, uint16_t *y);
int orc_block_values_f64(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                         int64_t cols, int blocking, double *out);

/* MXFP4 (32-element blocks, E8M0 scale; see the source for the rule). */
uint8_t orc_mx_scale(float amax);
double orc_mx_scale_value(uint8_t s);
int orc_mx_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                    uint8_t *codes, uint8_t *scales, uint32_t *status);
int orc_mx_block_values_f64(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                            int64_t cols, double *out);

void orc_f32_to_bf16_array(const float *f, int64_t n, uint16_t *out);
void orc_e4m3_encode_array(const float *s, int64_t n, uint8_t *out);
void orc_e2m1_encode_rn_array(const float *v, int64_t n, uint8_t *out);
void orc_e2m1_encode_sr_array(const float *v, const uint16_t *k, int64_t n, uint8_t *out);
void orc_philox_array(const uint32_t *ctr, const uint32_t *key, int64_t n, uint32_t *out);
void orc_sr_bits_array(uint64_t seed, uint64_t first, int64_t n, uint16_t *out);
void orc_rht16_rows(const float *x, int64_t ngroups, uint64_t seed, float *y);
void orc_rht16_rows_signs(const float *x, int64_t ngroups, const float d[16], float *y);
int orc_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
