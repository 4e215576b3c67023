// quantize.hip -- NVFP4 quantization kernels for gfx950.
//
// Recipe (NVIDIA developer blog zh-cn "NVFP4 trains with precision of 16-bit ...",
// section "用于预训练的 NVFP4 量化配方"; prism.simon-ai.net article 7890, sections
// "MVFP4格式的核心架构革新", "训练稳定性与敏感层保护策略", "应对异常值与舍入误差的技术手段"):
// optional 16-point random Hadamard transform per 16-element row group, an FP32 tensor
// scale from the tensor amax, an E4M3 scale per 1x16 or 16x16 block, E2M1 codes by
// nearest-even or stochastic rounding (Philox4x32-10 keyed on (seed, element index)).
//
// The tensor scale needs the amax of the whole (transformed) tensor before any code can
// be written, so quantization is two passes over the input:
//   pass 1  amax_kernel: each workgroup reduces a contiguous range of row groups to one
//           partial amax (integer max of |y| bit patterns: exact and order-free);
//   pass 2  quant_1x16_kernel / quant_16x16_kernel: every workgroup reduces the partials,
//           derives the tensor scales on the device (no host sync), and encodes its range.
// Pass 2 re-reads an input that pass 1 has just streamed, which the 256 MB Infinity
// Cache holds for the sizes this library targets.
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint32_t rht_signmask(uint32_t k0, uint32_t k1) {
  // Sign vector: bit j of word 0 of Philox4x32-10(key = seed, counter = (0, 0, 1, 0)).
  return philox4x32_10(0u, 0u, 1u, 0u, k0, k1).x & 0xFFFFu;
}

template <bool CONTIG>
__device__ __forceinline__ const uint4 *group_ptr(const uint16_t *x, uint32_t g, uint32_t gpr,
                                                  int64_t ld) {
  if (CONTIG) return reinterpret_cast<const uint4 *>(x + (size_t)g * 16u);
  const uint32_t r = g / gpr, gc = g - r * gpr;
  return reinterpret_cast<const uint4 *>(x + (size_t)r * (size_t)ld + (size_t)gc * 16u);
}

__device__ __forceinline__ uint32_t block_max_bits(uint32_t m) {
  __shared__ uint32_t red[kWaves];
  m = wave_max_u32(m);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = m;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = max(r, red[i]);
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------- pass 1
template <bool RHT, bool CONTIG>
__global__ __launch_bounds__(kThreads) void amax_kernel(const uint16_t *__restrict__ x,
                                                        uint32_t ngroups, uint32_t gpr,
                                                        int64_t ld, uint32_t rk0,
                                                        uint32_t rk1, uint32_t per_wg,
                                                        uint32_t *__restrict__ partials) {
  const uint32_t sm = RHT ? rht_signmask(rk0, rk1) : 0u;
  const uint32_t begin = blockIdx.x * per_wg;
  const uint32_t end = min(begin + per_wg, ngroups);
  uint32_t m = 0;
  constexpr int U = 4;   // row groups in flight per thread
  for (uint32_t g0 = begin + threadIdx.x; g0 < end; g0 += U * kThreads) {
    uint4 a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t g = g0 + u * kThreads;
      if (g < end) {
        const uint4 *p = group_ptr<CONTIG>(x, g, gpr, ld);
        a[u] = p[0];
        b[u] = p[1];
      } else {
        a[u] = make_uint4(0u, 0u, 0u, 0u);
        b[u] = a[u];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float v[16];
      unpack16(a[u], b[u], v);
      if (RHT) rht16(v, sm);
#pragma unroll
      for (int j = 0; j < 16; ++j) m = max(m, __float_as_uint(v[j]) & 0x7FFFFFFFu);
    }
  }
  m = block_max_bits(m);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// Reduce the partial maxima of pass 1 and publish the tensor scale (workgroup 0).
__device__ __forceinline__ TensorScale finish_amax(const uint32_t *__restrict__ partials,
                                                   uint32_t nparts, float *global_dec,
                                                   uint32_t *dev_status) {
  uint32_t m = 0;
  for (uint32_t i = threadIdx.x; i < nparts; i += kThreads) m = max(m, partials[i]);
  m = block_max_bits(m);
  const TensorScale ts = tensor_scale(m);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *global_dec = ts.dec;
    if (dev_status) *dev_status = ts.finite ? 0u : 1u;
  }
  return ts;
}

// Encode the 16 transformed values of one row group with the block multiplier rr.
// k[16]: 16-bit random integers (stochastic rounding only).
template <bool SR>
__device__ __forceinline__ uint2 encode16(const float y[16], float rr, const uint32_t k[16]) {
  if (!SR) return e2m1_rn_pack16(y, rr);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float a = fabsf(y[j] * rr);
    const uint32_t mag = SR ? e2m1_sr_mag(a, k[j]) : e2m1_rn_mag(a);
    const uint32_t q = mag | ((__float_as_uint(y[j]) >> 28) & 8u);
    if (j < 8) lo |= q << (4 * j);
    else hi |= q << (4 * (j - 8));
  }
  return make_uint2(lo, hi);
}

// The 16 random integers of elements idx0 .. idx0+15 (idx0 a multiple of 16): element i
// takes 16-bit lane (i & 7) of Philox4x32-10(key, counter = (i >> 3, 0, 0)).
__device__ __forceinline__ void sr_draws(uint64_t idx0, uint32_t k0, uint32_t k1,
                                         uint32_t k[16]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint64_t c = (idx0 >> 3) + (uint64_t)h;
    const Philox4 r = philox4x32_10((uint32_t)c, (uint32_t)(c >> 32), 0u, 0u, k0, k1);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) k[8 * h + j] = (w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
  }
}

__device__ __forceinline__ float absmax16(const float v[16]) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(v[j]));
  return m;
}

// ---------------------------------------------------------------- pass 2, 1x16
// One row group per thread per step; the next step's 32 input bytes are loaded before
// the current group is encoded, so every wave keeps a load in flight while it computes.
template <bool RHT, bool SR, bool CONTIG>
__global__ __launch_bounds__(kThreads) void quant_1x16_kernel(
    const uint16_t *__restrict__ x, uint32_t ngroups, uint32_t gpr, int64_t ld, int64_t cols,
    uint32_t rk0, uint32_t rk1, uint32_t sk0, uint32_t sk1, uint64_t sr_base, uint32_t per_wg,
    const uint32_t *__restrict__ partials, uint32_t nparts, uint8_t *__restrict__ codes,
    uint8_t *__restrict__ scales, float *__restrict__ global_dec, uint32_t *dev_status) {
  const uint32_t begin = blockIdx.x * per_wg;
  const uint32_t end = min(begin + per_wg, ngroups);
  uint32_t g = begin + threadIdx.x;
  // the first group's load is in flight while the tensor scale is reduced (an empty
  // tensor has no group to load: its workgroup only publishes the tensor scale)
  uint4 ca = make_uint4(0u, 0u, 0u, 0u), cb = ca;
  if (begin < end) {
    const uint4 *p = group_ptr<CONTIG>(x, g < end ? g : begin, gpr, ld);
    ca = p[0];
    cb = p[1];
  }
  const TensorScale ts = finish_amax(partials, nparts, global_dec, dev_status);
  if (!ts.finite) return;
  const uint32_t sm = RHT ? rht_signmask(rk0, rk1) : 0u;
  for (; g < end; g += kThreads) {
    // next group (on the last step this re-reads the current one: always a valid address)
    const uint32_t gn = g + kThreads < end ? g + kThreads : g;
    const uint4 *pn = group_ptr<CONTIG>(x, gn, gpr, ld);
    const uint4 na = pn[0], nb = pn[1];
    float v[16];
    unpack16(ca, cb, v);
    if (RHT) rht16(v, sm);
    const float bmax = absmax16(v);
    const uint32_t sb = e4m3_encode((bmax / kE2M1Max) * ts.enc);
    const float rr = block_mult(ts.enc, e4m3_decode(sb));
    uint32_t k[16];
    if (SR) {
      const uint32_t r = g / gpr, gc = g - r * gpr;
      sr_draws(sr_base + (uint64_t)r * (uint64_t)cols + (uint64_t)gc * 16u, sk0, sk1, k);
    }
    reinterpret_cast<uint2 *>(codes)[g] = encode16<SR>(v, rr, k);  // group g at byte 8g
    scales[g] = (uint8_t)sb;
    ca = na;
    cb = nb;
  }
}

// ---------------------------------------------------------------- pass 2, 16x16
// A workgroup encodes a block of 16 x 16 tiles (256 x 256 elements) in 16 steps, one
// tile-row of 16 tiles per step; 16 lanes of a DPP row hold the 16 rows of a tile.  The
// tile amax is a DPP max over the row.  Codes of x are stored per step (128 contiguous
// bytes per row); with TRANS the codes of x^T come from an in-register 4-bit transpose and
// are assembled in LDS so that each of the block's 256 rows of x^T is written as one
// 128-byte line at the end (a row of x^T receives 8 bytes per tile-row of x).
constexpr int kTStride = 136;   // LDS bytes per staged x^T row (128 + 8 against bank conflicts)

template <bool SR, bool TRANS>
__global__ __launch_bounds__(kThreads) void quant_16x16_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, int64_t ld, uint32_t sk0,
    uint32_t sk1, uint64_t sr_base, const uint32_t *__restrict__ partials, uint32_t nparts,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, uint8_t *__restrict__ codes_t,
    uint8_t *__restrict__ scales_t, float *__restrict__ global_dec, uint32_t *dev_status) {
  __shared__ __attribute__((aligned(16))) uint8_t tbuf[TRANS ? 256 * kTStride : 16];
  __shared__ __attribute__((aligned(16))) uint8_t sbuf[TRANS ? 256 : 16];
  const uint32_t tpr = (uint32_t)(cols >> 4);          // tiles per tile-row
  const uint32_t tpc = (uint32_t)(rows >> 4);          // tiles per tile-column
  if (tpr == 0 || tpc == 0) {   // empty tensor: only the tensor scale is written
    finish_amax(partials, nparts, global_dec, dev_status);
    return;
  }
  const uint32_t bpr = (tpr + 15) >> 4;                // blocks per block-row
  const uint32_t blk = blockIdx.x;
  const uint32_t br = blk / bpr, bc = blk - br * bpr;
  const uint32_t tl = threadIdx.x >> 4, r = threadIdx.x & 15u;
  const uint32_t tc = bc * 16 + tl;                    // this lane's tile column
  const bool col_ok = tc < tpr;
  // every lane loads a valid address (the block's first tile when past an edge) and
  // masks the data, so the 16 lanes of a tile always run the reductions together
  auto load = [&](uint32_t it, uint4 &a, uint4 &b) {
    const uint32_t tr = br * 16 + it;
    const bool valid = col_ok && tr < tpc;
    const uint32_t rr_ = valid ? tr : br * 16, cc = valid ? tc : bc * 16;
    const uint4 *p = reinterpret_cast<const uint4 *>(x + ((int64_t)rr_ * 16 + r) * ld + (int64_t)cc * 16);
    const uint4 ra = p[0], rb = p[1];
    const uint32_t m = valid ? 0xFFFFFFFFu : 0u;
    a = make_uint4(ra.x & m, ra.y & m, ra.z & m, ra.w & m);
    b = make_uint4(rb.x & m, rb.y & m, rb.z & m, rb.w & m);
  };
  uint4 ca, cb;
  load(0, ca, cb);                    // in flight while the tensor scale is reduced
  const TensorScale ts = finish_amax(partials, nparts, global_dec, dev_status);
  if (!ts.finite) return;
  const uint32_t nit = min(16u, tpc - br * 16);
  for (uint32_t it = 0; it < nit; ++it) {
    uint4 na, nb;
    load(it + 1 < nit ? it + 1 : it, na, nb);
    const uint32_t tr = br * 16 + it;
    const int64_t row = (int64_t)tr * 16 + r;
    float v[16];
    unpack16(ca, cb, v);
    const uint32_t tmax = row16_max_u32(__float_as_uint(absmax16(v)));
    const uint32_t sb = e4m3_encode((__uint_as_float(tmax) / kE2M1Max) * ts.enc);
    const float rr = block_mult(ts.enc, e4m3_decode(sb));
    uint32_t k[16];
    if (SR) sr_draws(sr_base + (uint64_t)row * (uint64_t)cols + (uint64_t)tc * 16u, sk0, sk1, k);
    uint2 q = encode16<SR>(v, rr, k);
    if (col_ok) {
      *reinterpret_cast<uint2 *>(codes + row * (cols >> 1) + (int64_t)tc * 8) = q;
      if (r == 0) scales[(size_t)tr * tpr + tc] = (uint8_t)sb;
    }
    if (TRANS) {
      transpose_nibbles16(q.x, q.y, r);   // lane r now holds column r of the tile
      *reinterpret_cast<uint2 *>(tbuf + (tl * 16 + r) * kTStride + it * 8) = q;
      if (r == 0) sbuf[tl * 16 + it] = (uint8_t)sb;
    }
    ca = na;
    cb = nb;
  }
  if (TRANS) {
    __syncthreads();
    // 256 staged rows of x^T, nit * 8 bytes each: row j of the block is x^T row
    // bc*256 + j, bytes [br*128, br*128 + 8*nit)
    const uint32_t nbytes = nit * 8;
    for (uint32_t i = threadIdx.x; i < 256 * 16; i += kThreads) {
      const uint32_t j = i >> 4, c8 = i & 15u;     // row, 8-byte chunk
      const uint32_t ttc = bc * 16 + (j >> 4);
      if (ttc < tpr && c8 * 8 < nbytes) {
        const uint2 w = *reinterpret_cast<const uint2 *>(tbuf + j * kTStride + c8 * 8);
        const int64_t trow = (int64_t)bc * 256 + j;
        *reinterpret_cast<uint2 *>(codes_t + trow * (rows >> 1) + (int64_t)br * 128 + c8 * 8) = w;
      }
    }
    // scales of x^T: row tc (one per tile column), bytes [br*16, br*16 + nit)
    if (threadIdx.x < 256) {
      const uint32_t tcl = threadIdx.x >> 4, it = threadIdx.x & 15u;
      const uint32_t ttc = bc * 16 + tcl;
      if (ttc < tpr && it < nit) scales_t[(size_t)ttc * tpc + br * 16 + it] = sbuf[tcl * 16 + it];
    }
  }
}

uint32_t ceil_div(uint64_t a, uint64_t b) { return (uint32_t)((a + b - 1) / b); }

// Workgroup caps of the encode pass (8 resident 256-thread workgroups per CU).
#ifndef NVFP4_Q1_MAX_WG
#define NVFP4_Q1_MAX_WG 2048
#endif
#ifndef NVFP4_AMAX_MAX_WG
#define NVFP4_AMAX_MAX_WG 1024
#endif

}  // namespace

hipError_t launch_quantize(const QuantLaunch &q, hipStream_t stream) {
  const uint64_t ngroups64 = (uint64_t)q.rows * (uint64_t)(q.cols / 16);
  const uint32_t ngroups = (uint32_t)ngroups64;
  const uint32_t gpr = (uint32_t)(q.cols / 16);
  const bool contig = (q.ld == q.cols);
  // pass 1 geometry: up to 1024 workgroups, each a contiguous range of row groups
  uint32_t nparts = ceil_div(ngroups64 ? ngroups64 : 1, kThreads * 4);
  if (nparts > NVFP4_AMAX_MAX_WG) nparts = NVFP4_AMAX_MAX_WG;
  const uint32_t per_wg = ceil_div(ngroups64 ? ngroups64 : 1, nparts);
  const bool rht = q.rht != 0;
#define NVFP4_AMAX(R, C)                                                                    \
  amax_kernel<R, C><<<nparts, kThreads, 0, stream>>>(q.x, ngroups, gpr, q.ld, q.rht_k0,    \
                                                     q.rht_k1, per_wg, q.partials)
  if (rht && contig) NVFP4_AMAX(true, true);
  else if (rht) NVFP4_AMAX(true, false);
  else if (contig) NVFP4_AMAX(false, true);
  else NVFP4_AMAX(false, false);
#undef NVFP4_AMAX

  if (q.blocking == 0) {
    const bool sr = q.rounding == 1;
    // pass 2 grid: enough workgroups for 8 per CU, each a contiguous range of groups
    uint32_t grid2 = ceil_div(ngroups64 ? ngroups64 : 1, kThreads);
    if (grid2 > NVFP4_Q1_MAX_WG) grid2 = NVFP4_Q1_MAX_WG;
    const uint32_t per_wg2 = ceil_div(ngroups64 ? ngroups64 : 1, grid2);
    grid2 = ceil_div(ngroups64 ? ngroups64 : 1, per_wg2);
#define NVFP4_Q1(R, S, C)                                                                   \
  quant_1x16_kernel<R, S, C><<<grid2, kThreads, 0, stream>>>(                               \
      q.x, ngroups, gpr, q.ld, q.cols, q.rht_k0, q.rht_k1, q.sr_k0, q.sr_k1, q.sr_base,     \
      per_wg2, q.partials, nparts, q.codes, q.scales, q.global_dec, q.dev_status)
    if (rht) {
      if (sr) { if (contig) NVFP4_Q1(true, true, true); else NVFP4_Q1(true, true, false); }
      else { if (contig) NVFP4_Q1(true, false, true); else NVFP4_Q1(true, false, false); }
    } else {
      if (sr) { if (contig) NVFP4_Q1(false, true, true); else NVFP4_Q1(false, true, false); }
      else { if (contig) NVFP4_Q1(false, false, true); else NVFP4_Q1(false, false, false); }
    }
#undef NVFP4_Q1
  } else {
    // one workgroup per block of 16 x 16 tiles
    uint32_t grid = (uint32_t)(((q.rows / 16 + 15) / 16) * ((q.cols / 16 + 15) / 16));
    if (grid == 0) grid = 1;   // an empty tensor still publishes its tensor scale
    const bool sr = q.rounding == 1, tr = q.codes_t != nullptr;
#define NVFP4_Q16(S, T)                                                                     \
  quant_16x16_kernel<S, T><<<grid, kThreads, 0, stream>>>(                                  \
      q.x, q.rows, q.cols, q.ld, q.sr_k0, q.sr_k1, q.sr_base, q.partials, nparts, q.codes,  \
      q.scales, q.codes_t, q.scales_t, q.global_dec, q.dev_status)
    if (sr) { if (tr) NVFP4_Q16(true, true); else NVFP4_Q16(true, false); }
    else { if (tr) NVFP4_Q16(false, true); else NVFP4_Q16(false, false); }
#undef NVFP4_Q16
  }
  return hipGetLastError();
}

}  // namespace nvfp4
