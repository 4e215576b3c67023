/*
 * nvfp4.h -- C ABI of libnvfp4: NVFP4 block-scaled FP4 quantization for AMD MI355X (gfx950).
 *
 * The format and the recipe come from these pages (cited by page and section):
 *   [NV-blog] developer.nvidia.com zh-cn blog "NVFP4 trains with precision of 16-bit and
 *             speed and efficiency of 4-bit", section "用于预训练的 NVFP4 量化配方", five
 *             bullets: 16-element micro-blocks, E4M3 block scales, Hadamard transform on
 *             GEMM inputs, selective 2D block quantization, stochastic rounding.
 *   [PR]      prism.simon-ai.net article 7890: section "MVFP4格式的核心架构革新" (an FP32
 *             per-tensor scale on top of the E4M3 block scales), "训练稳定性与敏感层保护策略"
 *             (16x16 blocks for weights so W and W^T agree), "应对异常值与舍入误差的技术手段"
 *             (random Hadamard transform keeps norms; stochastic rounding of gradients).
 *
 * Conventions for every call:
 *   - Pointers marked (device) are HIP device memory; (host) is host memory.  The caller
 *     owns every buffer.  The library never allocates, never synchronizes and keeps no
 *     global state: all calls are re-entrant and asynchronous on `stream`.
 *   - Argument errors are returned before any HIP call is made.  A failed kernel launch
 *     returns NVFP4_ERR_HIP.  Errors that depend on the data (inf/NaN input) are reported
 *     on the device: the tensor scale becomes NaN and *dev_status becomes nonzero.
 *   - Every device pointer must be 16-byte aligned; leading dimensions are in elements.
 *   - Data pointers of an empty tensor (a zero dimension) may be NULL; the tensor scale
 *     output of nvfp4_quantize is still written (1.0).
 *   - `stream` is a hipStream_t (NULL = the default stream).
 *
 * Storage (identical for inputs and outputs of all calls):
 *   codes   packed E2M1, two per byte, row-major, rows x cols/2 bytes; column 2j in the
 *           low nibble, column 2j+1 in the high nibble.  Nibble = sign<<3 | exp<<1 | man
 *           (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6).
 *   scales  E4M3 (OCP E4M3FN, max 448), row-major:
 *             NVFP4_BLOCK_1x16 : rows    x cols/16 bytes (one per 16 consecutive elements
 *                                of a row),
 *             NVFP4_BLOCK_16x16: rows/16 x cols/16 bytes (one per 16x16 tile).
 *   global  one float: the decode scale s_dec = amax / (6 * 448) of the (transformed)
 *           tensor; 1.0 for an all-zero tensor; NaN if the input held inf or NaN.
 *   A value decodes as e2m1(code) * e4m3(scale) * global.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 1

struct ihipStream_t;
typedef struct ihipStream_t *nvfp4_stream_t; /* same type as hipStream_t */

typedef enum {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL = 1,        /* a required pointer is NULL */
    NVFP4_ERR_SHAPE = 2,       /* a size is negative or not a multiple of 16, or ld too small */
    NVFP4_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned or ld not a multiple of 8 */
    NVFP4_ERR_UNSUPPORTED = 4, /* an option combination this version does not implement */
    NVFP4_ERR_WORKSPACE = 5,   /* workspace missing or smaller than the *_workspace_bytes value */
    NVFP4_ERR_HIP = 6          /* a HIP launch failed */
} nvfp4_status;

typedef enum { NVFP4_BLOCK_1x16 = 0, NVFP4_BLOCK_16x16 = 1 } nvfp4_blocking;
typedef enum { NVFP4_ROUND_RNE = 0, NVFP4_ROUND_STOCHASTIC = 1 } nvfp4_rounding;
typedef enum { NVFP4_OUT_BF16 = 0, NVFP4_OUT_FP32 = 1 } nvfp4_out_dtype;

/* Quantization options (host struct). */
typedef struct {
    int32_t blocking;       /* nvfp4_blocking: 1x16 for activations and gradients, 16x16
                               for weights ([NV-blog] bullets 1 and 4; [PR] training
                               stability section) */
    int32_t rounding;       /* nvfp4_rounding: nearest-even, or stochastic ([NV-blog]
                               bullet 5; [PR] outliers-and-rounding section) */
    int32_t rht;            /* 1: apply the 16-point random Hadamard transform to every
                               16-element row group before quantizing ([NV-blog] bullet 3),
                               with either blocking.  Quantizing a GEMM's two K-contiguous
                               operands with the same rht_seed keeps their product ([PR]
                               outliers section: dot products are unchanged) */
    int32_t reserved;       /* must be 0 */
    uint64_t rht_seed;      /* selects the +-1 sign vector of the transform */
    uint64_t sr_seed;       /* Philox4x32-10 key for stochastic rounding */
    uint64_t sr_index_base; /* Philox element index of x[0][0]; a multiple of 16.  Lets a
                               tensor be quantized in row chunks with the same draws as
                               one call over the whole tensor */
} nvfp4_quant_params;

/* NVFP4 operand of the GEMM (device pointers): rows x K, K contiguous. */
typedef struct {
    const uint8_t *codes;     /* rows x K/2 bytes */
    const uint8_t *scales;    /* E4M3 scales in the layout of `blocking` */
    const float *global_dec;  /* 1 float (device) */
    int32_t blocking;         /* nvfp4_blocking */
    int32_t reserved;         /* must be 0 */
} nvfp4_operand;

/* Bytes of device memory nvfp4_quantize needs as its workspace (caller-allocated; the same
 * value for every shape the ABI accepts).  The workspace carries coordination state from
 * one call to the next: zero-fill it once before its first use and then leave it to the
 * library.  A workspace serves one stream: calls that use it must not overlap in time. */
size_t nvfp4_quantize_workspace_bytes(void);

/*
 * nvfp4_quantize -- quantize a row-major bf16 tensor to NVFP4.
 *
 * Computes, per [NV-blog] bullets 1-5 and [PR] "MVFP4格式的核心架构革新":
 *   y      = x, or RHT16(x) along each 16-element row group (if p->rht);
 *   amax   = max |y| over the tensor; s_enc = 2688 / amax; global = amax / 2688;
 *   per block (1x16 or 16x16): sb = e4m3((max|y| / 6) * s_enc), nearest-even, at most 448;
 *   per element: code = e2m1(y * (s_enc / e4m3_decode(sb))), nearest-even or stochastic
 *   (Philox4x32-10 keyed on (sr_seed, element index)); the code keeps the sign of y.
 *
 * x           (device) bf16 bit patterns, rows x cols, row stride ld_x >= cols elements.
 * rows, cols  multiples of 16 (0 is allowed and does nothing).
 * p           (host) options; not retained.
 * codes       (device, out) rows x cols/2 bytes.
 * scales      (device, out) see Storage.
 * global_dec  (device, out) 1 float.
 * codes_t     (device, out, optional; 16x16 only) codes of x^T: cols x rows/2 bytes.  With
 *             16x16 blocks these are exactly the transposed codes of x, so W and W^T come
 *             from one read ([PR] training stability section).  NULL to skip.
 * scales_t    (device, out) scales of x^T, cols/16 x rows/16; required iff codes_t is given.
 * dev_status  (device, out, optional) 0; 1 if the input held inf or NaN; 2 if a wait
 *             between workgroups passed its last-resort time limit (the results are then
 *             invalid; this indicates a fault, not a property of the input).
 * workspace   (device) at least nvfp4_quantize_workspace_bytes() bytes, zero-filled before
 *             its first use (see nvfp4_quantize_workspace_bytes).  Calls captured in a
 *             HIP graph may be replayed: each launch tags its state afresh.
 */
nvfp4_status nvfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                            const nvfp4_quant_params *p, uint8_t *codes, uint8_t *scales,
                            float *global_dec, uint8_t *codes_t, uint8_t *scales_t,
                            uint32_t *dev_status, void *workspace, size_t workspace_bytes,
                            nvfp4_stream_t stream);

/*
 * nvfp4_quantize_noalloc -- nvfp4_quantize without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The library keeps the workspace in a file-scope device
 * array of nvfp4_quantize_workspace_bytes() bytes (8 MiB + 12 KiB), one per GPU, held until
 * the process ends; it covers every shape the ABI accepts.  The call allocates nothing.
 *
 * Arguments, results and errors as nvfp4_quantize, without workspace/workspace_bytes.  The
 * array is found on the device of `stream`; its address is looked up once per device (the
 * first call on a device makes that HIP call; a failure returns NVFP4_ERR_HIP).
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU
 * (several streams or host threads) race and must not be made; calls in stream order,
 * graph replays included, are fine.
 */
nvfp4_status nvfp4_quantize_noalloc(const uint16_t *x, int64_t rows, int64_t cols,
                                    int64_t ld_x, const nvfp4_quant_params *p, uint8_t *codes,
                                    uint8_t *scales, float *global_dec, uint8_t *codes_t,
                                    uint8_t *scales_t, uint32_t *dev_status,
                                    nvfp4_stream_t stream);

/*
 * nvfp4_dequantize -- y = e2m1(code) * e4m3(scale) * global ([PR] "MVFP4与MXFP4": a 4-bit
 * value times its block scale gives the real value; "MVFP4格式的核心架构革新": the FP32
 * tensor scale on top).  The first product is exact; bf16 output rounds the fp32 value
 * to nearest-even.
 *
 * codes, scales, global_dec  (device) as produced by nvfp4_quantize with `blocking`.
 * y          (device, out) rows x cols, row stride ld_y >= cols elements (multiple of 8),
 *            bf16 bit patterns or float per `out_dtype`.
 */
nvfp4_status nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales,
                              const float *global_dec, int64_t rows, int64_t cols,
                              int32_t blocking, void *y, int64_t ld_y, int32_t out_dtype,
                              nvfp4_stream_t stream);

/*
 * nvfp4_gemm -- C = A . B^T for NVFP4 operands, fp32 accumulation.
 *
 * The linear-layer matrix product the recipe accelerates ([NV-blog] recipe section,
 * Figure 1 paragraph: LLMs rest on the matrix products of their linear layers).
 *   C[m][n] = gA * gB * sum_k (e2m1 * e4m3)_A[m][k] * (e2m1 * e4m3)_B[n][k]
 * a  (host struct, device pointers) M x K operand (activations; any blocking).
 * b  (host struct, device pointers) N x K operand, i.e. the transposed weight W^T (with
 *    16x16 blocks, the codes_t/scales_t of a K x N weight, or a weight quantized as N x K).
 * M, N, K  multiples of 16; M, N <= 2^30, K <= 2^23, and at most 2^31 - 1 tiles of
 *          128 x 128 in C.
 * c  (device, out) M x N row-major, row stride ldc >= N (multiple of 8), bf16 or float.
 */
nvfp4_status nvfp4_gemm(const nvfp4_operand *a, const nvfp4_operand *b, int64_t M, int64_t N,
                        int64_t K, void *c, int64_t ldc, int32_t out_dtype,
                        nvfp4_stream_t stream);

/* Bytes of device memory nvfp4_gemm_ws needs as its workspace (caller-allocated; the same
 * value for every shape): 4 KiB of counters and 256 fp32 partial tiles of 256 x 256. */
size_t nvfp4_gemm_workspace_bytes(void);

/*
 * nvfp4_gemm_ws -- the product of nvfp4_gemm ([NV-blog] recipe section, Figure 1
 * paragraph), with a workspace.  The GEMM runs one 256 x 256 tile per compute unit at a
 * time; when the tile count is not a multiple of the compute units, the tiles of the last
 * round are split along K over otherwise idle units, their fp32 partial tiles summed in
 * the workspace in a fixed order (the result does not depend on scheduling, but may differ
 * from nvfp4_gemm's in the last bits: the K sum is associated differently).
 * Arguments as nvfp4_gemm, and:
 * workspace        (device) at least nvfp4_gemm_workspace_bytes() bytes, 16-byte aligned,
 *                  zero-filled before its first use; every call leaves its counters at zero
 *                  again.  A workspace serves one stream: calls that use it must not overlap.
 * workspace_bytes  its size.
 * Errors: as nvfp4_gemm; NVFP4_ERR_WORKSPACE for a NULL or short workspace.
 */
nvfp4_status nvfp4_gemm_ws(const nvfp4_operand *a, const nvfp4_operand *b, int64_t M, int64_t N,
                           int64_t K, void *c, int64_t ldc, int32_t out_dtype, void *workspace,
                           size_t workspace_bytes, nvfp4_stream_t stream);

/*
 * nvfp4_transpose_bf16 -- y = x^T for a bf16 tensor (bit patterns are moved, not changed).
 * The weight-gradient GEMM of a linear layer contracts over the token dimension
 * ([NV-blog] recipe section, bullet 3: the transform and the quantization apply to the GEMM
 * inputs of the backward pass too), so X^T and dY^T are quantized along it: this call lays
 * them out with that dimension contiguous.
 * x     (device) rows x cols, row stride ld_x >= cols (multiple of 8).
 * rows, cols  multiples of 8.
 * y     (device, out) cols x rows, row stride ld_y >= rows (multiple of 8).
 */
nvfp4_status nvfp4_transpose_bf16(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                                  uint16_t *y, int64_t ld_y, nvfp4_stream_t stream);

/* ------------------------------------------------------------------------------------
 * MXFP4: the format the pages compare NVFP4 with ([NV-blog] recipe section, bullets 1-2:
 * 32-element blocks with a power-of-two E8M0 scale instead of 16 with E4M3; [PR]
 * "MVFP4与MXFP4"), the block format gfx950's scaled FP4 matrix instructions consume.
 * The pages do not say how the power of two is picked; these calls use the OCP
 * Microscaling Formats v1.0 rule: X = 2^(floor(log2 amax) - 2) over the block's finite
 * amax (2 = exponent of E2M1's largest value 6), clamped to [2^-127, 2^127], biased byte
 * s = log2 X + 127 (an all-zero block gets s = 0); a block holding inf or NaN gets the NaN
 * scale s = 0xFF and zero codes.  Element code = e2m1(x / X), nearest-even, saturating at
 * +-6, keeping the sign (also of zero).  There is no tensor scale and no status output:
 * a non-finite block is visible as its 0xFF scale.
 *
 * Storage: codes as for NVFP4 (rows x cols/2 bytes, column 2j in the low nibble); scales
 * rows x cols/32 bytes, row-major, one per 32 consecutive elements of a row.  A value
 * decodes as e2m1(code) * 2^(s - 127) (NaN if s = 0xFF).
 * ---------------------------------------------------------------------------------- */

/*
 * mxfp4_quantize -- quantize a row-major bf16 tensor to MXFP4 (rule above).
 * x       (device) bf16 bit patterns, rows x cols, row stride ld_x >= cols (multiple of 8).
 * rows    >= 0; cols a multiple of 32; rows * cols <= 2^34.
 * codes   (device, out) rows x cols/2 bytes.   scales (device, out) rows x cols/32 bytes.
 */
nvfp4_status mxfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                            uint8_t *codes, uint8_t *scales, nvfp4_stream_t stream);

/*
 * mxfp4_dequantize -- y = e2m1(code) * 2^(s - 127), exact in both output types (NaN for
 * s = 0xFF; e2m1 6 with s >= 254 overflows to inf).
 * codes, scales  (device) in the MXFP4 storage above.
 * y       (device, out) rows x cols, row stride ld_y >= cols (multiple of 8), bf16 or float.
 */
nvfp4_status mxfp4_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                              int64_t cols, void *y, int64_t ld_y, int32_t out_dtype,
                              nvfp4_stream_t stream);

/*
 * mxfp4_gemm -- C = A . B^T for MXFP4 operands on the native scaled FP4 matrix
 * instructions, fp32 accumulation (the product of the NVFP4 GEMM, with 32-element E8M0
 * blocks and no tensor scales).
 *   C[m][n] = sum_k e2m1(A[m][k]) 2^(sA[m][k/32] - 127) * e2m1(B[n][k]) 2^(sB[n][k/32] - 127)
 * a_codes, a_scales  (device) M x K operand.   b_codes, b_scales (device) N x K operand.
 * M, N in [0, 2^24], at most 2^31 - 1 tiles of 128 x 128 in C; K a multiple of 32, at
 * most 2^23.
 * c       (device, out) M x N row-major, row stride ldc >= N (any), bf16 or float.
 */
nvfp4_status mxfp4_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                        const uint8_t *b_scales, int64_t M, int64_t N, int64_t K, void *c,
                        int64_t ldc, int32_t out_dtype, nvfp4_stream_t stream);

/* Static, NUL-terminated description of a status code. */
const char *nvfp4_status_string(nvfp4_status s);

/* NVFP4_ABI_VERSION of the built library. */
int nvfp4_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_H */
