// gemm.hip -- NVFP4 x NVFP4 GEMM on gfx950 matrix cores.
//
// C[m][n] = gA * gB * sum_k (e2m1 * e4m3)_A[m][k] * (e2m1 * e4m3)_B[n][k]
// The linear-layer product the recipe exists to accelerate (NVIDIA developer blog zh-cn
// "NVFP4 trains with precision of 16-bit ...", section "用于预训练的 NVFP4 量化配方", the
// Figure 1 paragraph on GEMM throughput).
//
// gfx950's FP4 matrix instructions apply power-of-two (E8M0) scales per 32 K-elements;
// NVFP4 carries an E4M3 scale per 16, whose mantissa cannot be folded into them.  Every
// product e2m1 * e4m3 is exactly representable in fp16 (at most 6 significant bits,
// magnitudes in [2^-10, 2688]), so each tile is dequantized exactly to fp16 in registers
// and fed to v_mfma_f32_32x32x16_f16 with fp32 accumulation; the two tensor scales are
// applied once in the epilogue.
//
// Tiling: 128 x 128 output tile per 256-thread workgroup (2 x 2 waves of 64 x 64, each
// 2 x 2 MFMA blocks of 32 x 32), K step 64.  Packed codes (4 bits per element) and
// scale bytes are staged in LDS; each lane dequantizes its own MFMA operands from LDS.
// Within a 64-wide K step, lane half h (lane / 32) supplies K elements 32h .. 32h+31 in
// four MFMA steps of 8; A and B use the same lane-to-K map, so each MFMA still pairs
// equal k on both sides and the four steps cover the 64 elements once.
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLdsStride = 48;       // LDS bytes per staged row (32 + 16 padding)

struct GemmParams {
  const uint8_t *ac, *as;
  const float *ag;
  const uint8_t *bc, *bs;
  const float *bg;
  int a16, b16;  // 1: 16x16 blocking (scale row = row / 16)
  int M, N, K;
  int64_t ldc;
  void *c;
};

// 16 packed bytes (32 elements) starting at K element kk of a row; `left` = K - kk.
template <bool K32>
__device__ __forceinline__ uint4 load_chunk(const uint8_t *p, int left) {
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (left >= 32) {
    if (K32) {
      v = *reinterpret_cast<const uint4 *>(p);
    } else {
      const uint2 a = reinterpret_cast<const uint2 *>(p)[0];
      const uint2 b = reinterpret_cast<const uint2 *>(p)[1];
      v = make_uint4(a.x, a.y, b.x, b.y);
    }
  } else if (left >= 16) {
    const uint2 a = *reinterpret_cast<const uint2 *>(p);
    v.x = a.x;
    v.y = a.y;
  }
  return v;
}

template <bool F32, bool K32>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[kBM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint8_t sB[kBN * kLdsStride];
  __shared__ uint8_t sAs[kBM * 4], sBs[kBN * 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, l32 = lane & 31;
  // one-dimensional grid (a y dimension would cap M at 65535 tiles)
  const int m0 = (int)(blockIdx.x / tiles_n) * kBM, n0 = (int)(blockIdx.x % tiles_n) * kBN;
  const int64_t rowb = p.K >> 1;
  const int kgroups = p.K >> 4;

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  for (int k0 = 0; k0 < p.K; k0 += kBK) {
    {  // codes: thread -> (row tid/2, 16-byte chunk tid%2)
      const int row = tid >> 1, ch = tid & 1, kk = k0 + 32 * ch;
      uint4 va = make_uint4(0u, 0u, 0u, 0u), vb = va;
      if (m0 + row < p.M) va = load_chunk<K32>(p.ac + (int64_t)(m0 + row) * rowb + (kk >> 1), p.K - kk);
      if (n0 + row < p.N) vb = load_chunk<K32>(p.bc + (int64_t)(n0 + row) * rowb + (kk >> 1), p.K - kk);
      *reinterpret_cast<uint4 *>(sA + row * kLdsStride + 16 * ch) = va;
      *reinterpret_cast<uint4 *>(sB + row * kLdsStride + 16 * ch) = vb;
    }
    {  // scales: threads 0..127 -> A rows, 128..255 -> B rows; 4 K-groups each
      const int row = tid & 127;
      const bool isb = tid >= 128;
      const int grow = (isb ? n0 : m0) + row;
      const bool rv = grow < (isb ? p.N : p.M);
      const uint8_t *sp = isb ? p.bs : p.as;
      const int srow = (isb ? p.b16 : p.a16) ? (grow >> 4) : grow;
      uint8_t *dst = isb ? sBs : sAs;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kg = (k0 >> 4) + j;
        dst[row * 4 + j] = (rv && kg < kgroups) ? sp[(int64_t)srow * kgroups + kg] : (uint8_t)0;
      }
    }
    __syncthreads();

    half8_t aop[2][4], bop[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = wm * 64 + i * 32 + l32;
      const uint4 c = *reinterpret_cast<const uint4 *>(sA + row * kLdsStride + 16 * h);
      const _Float16 s0 = (_Float16)e4m3_decode(sAs[row * 4 + 2 * h]);
      const _Float16 s1 = (_Float16)e4m3_decode(sAs[row * 4 + 2 * h + 1]);
      aop[i][0] = dequant8_f16(c.x, s0);
      aop[i][1] = dequant8_f16(c.y, s0);
      aop[i][2] = dequant8_f16(c.z, s1);
      aop[i][3] = dequant8_f16(c.w, s1);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = wn * 64 + j * 32 + l32;
      const uint4 c = *reinterpret_cast<const uint4 *>(sB + row * kLdsStride + 16 * h);
      const _Float16 s0 = (_Float16)e4m3_decode(sBs[row * 4 + 2 * h]);
      const _Float16 s1 = (_Float16)e4m3_decode(sBs[row * 4 + 2 * h + 1]);
      bop[j][0] = dequant8_f16(c.x, s0);
      bop[j][1] = dequant8_f16(c.y, s0);
      bop[j][2] = dequant8_f16(c.z, s1);
      bop[j][3] = dequant8_f16(c.w, s1);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[i][s], bop[j][s], acc[i][j], 0, 0, 0);
    __syncthreads();
  }

  const float alpha = (*p.ag) * (*p.bg);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int col = n0 + wn * 64 + j * 32 + l32;
        if (row < p.M && col < p.N) {
          const float v = acc[i][j][r] * alpha;
          if (F32) {
            reinterpret_cast<float *>(p.c)[(int64_t)row * p.ldc + col] = v;
          } else {
            const uint32_t u = __float_as_uint(v);
            const uint32_t b = ((u & 0x7FFFFFFFu) > 0x7F800000u) ? ((u >> 16) | 0x40u)
                                                                : ((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
            reinterpret_cast<uint16_t *>(p.c)[(int64_t)row * p.ldc + col] = (uint16_t)b;
          }
        }
      }
}

// ---------------------------------------------------------------- 256 x 256 tiles
// Main path for K % 256 == 0.  One 256-thread workgroup per CU computes a 256 x 256 tile;
// each wave owns 128 x 128 (4 x 4 MFMA blocks, 256 fp32 accumulators).  K advances 256
// elements per step: every row of A and B contributes one 128-byte cache line of packed
// codes and 16 scale bytes, which the direct global->LDS loads (buffer_load ... lds)
// bring into one of two LDS stages while the waves compute on the other.  The 16-byte
// chunks of a row are stored at slot (chunk ^ ((row >> 1) & 7)): a 128-bit LDS read serves
// 16 lanes (16 consecutive rows) per pass, and with 128-byte rows the 16 (row parity,
// slot) pairs then cover the 64 banks once.  Scales are stored as [dword j][row] (4 bytes
// per row per 64 K-elements), so the 32 rows a wave reads together are 32 consecutive
// dwords.
//
// K mapping inside a step: lane half h reads chunk 2j + h (32 elements) for j = 0..3 and
// feeds its 8-element pieces to four MFMAs; A and B use the same map.
typedef int v4i32 __attribute__((ext_vector_type(4)));
constexpr int kT2 = 256;                 // tile rows (M) and columns (N)
constexpr int kRowB2 = 128;              // packed bytes per row per K step (256 elements)
constexpr int kCodesB2 = kT2 * kRowB2;   // 32 KB per operand per stage
constexpr int kScalesB2 = kT2 * 16;      // 4 KB per operand per stage
constexpr int kStageB2 = 2 * kCodesB2 + 2 * kScalesB2;

__device__ __forceinline__ uint4 lds16(const uint8_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// Work items.  Workgroups 0 .. t_dp-1 each compute one whole tile (t_dp is all tiles, or
// the tiles of the full rounds when the last round would leave CUs idle).  With a
// workspace, each remaining tile is split along K into `splits` contiguous ranges of K
// steps, one workgroup each: every split item stores its fp32 partial tile in the
// workspace and counts itself on the tile's counter; the last to arrive sums the
// partials in split order (so the result does not depend on arrival order), resets the
// counter and runs the epilogue.  No workgroup waits for another.
template <bool F32>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void gemm256_kernel(GemmParams p, int tiles_m, int tiles_n, int t_dp, int splits, uint8_t *ws) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kStageB2];
  __shared__ uint32_t sk_last;

  // tile order: the workgroups that one XCD (block id % 8) runs form a contiguous
  // range of tiles, walked four tile-rows at a time so concurrent tiles share A and B
  const int nk_all = p.K / 256;
  int b = blockIdx.x, item = -1, kbeg = 0, kend = nk_all;
  if (b < t_dp) {
    if ((t_dp & 7) == 0) b = (b & 7) * (t_dp >> 3) + (b >> 3);
  } else {
    item = b - t_dp;
    const int sp = item % splits;
    b = t_dp + item / splits;
    kbeg = (int)((int64_t)sp * nk_all / splits);
    kend = (int)((int64_t)(sp + 1) * nk_all / splits);
  }
  const int gm = 4;
  const int band = b / (gm * tiles_n), in_band = b - band * gm * tiles_n;
  const int rows_in_band = min(gm, tiles_m - band * gm);
  const int tm = band * gm + in_band % rows_in_band;
  const int tn = in_band / rows_in_band;
  const int m0 = tm * kT2, n0 = tn * kT2;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t rowb = p.K >> 1;
  const int kgroups = p.K >> 4;
  const int nk = kend - kbeg;   // K steps of this work item, from step kbeg

  // Tiles travel through registers: bounds-checked 16-byte buffer loads (a row past the
  // end of an operand reads zeros, and zero codes and scales contribute nothing; those
  // rows are not stored) early in a K step, LDS writes after the stage barrier.  Load i
  // of wave w covers tile row 64w + 8i + lane/8, natural chunk lane%8, which goes to
  // slot chunk ^ ((row >> 1) & 7) = chunk ^ (4 (i & 1) + lane/16).  (The direct
  // global->LDS load instructions were measured to cost ~250 cycles of issue each here.)
  // The resources start at the tile's first row and end at the operand's last, so offsets
  // stay below 256 rows (32-bit for K < 2^24) however large the operands are.  The whole
  // offset of every load is the per-lane offset (the scalar offset is zero): the range
  // check, which covers the per-lane offset, then sees a row's full address, and a row past
  // the operand's end is never read.
  const int rows_a = min(p.M - m0, kT2), rows_b = min(p.N - n0, kT2);
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(p.ac + (int64_t)m0 * rowb, (int64_t)rows_a * rowb);
  const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(p.bc + (int64_t)n0 * rowb, (int64_t)rows_b * rowb);
  const int64_t s0a = p.a16 ? (m0 >> 4) : m0, s0b = p.b16 ? (n0 >> 4) : n0;
  const int64_t snra = p.a16 ? (rows_a + 15) / 16 : rows_a, snrb = p.b16 ? (rows_b + 15) / 16 : rows_b;
  const __amdgpu_buffer_rsrc_t rsa = buffer_rsrc(p.as + s0a * kgroups, snra * kgroups);
  const __amdgpu_buffer_rsrc_t rsb = buffer_rsrc(p.bs + s0b * kgroups, snrb * kgroups);
  const int voff_code = (int)((64 * wave + (lane >> 3)) * rowb + (lane & 7) * 16);
  const int wr_e = (lane >> 3) * kRowB2 + (((lane & 7) ^ (lane >> 4)) * 16);
  const int wr_o = (lane >> 3) * kRowB2 + (((lane & 7) ^ (4 + (lane >> 4))) * 16);
  const int srow = 64 * wave + lane;   // scale rows: wave w loads tile rows 64w .. 64w+63
  const int voff_sa = (int)((p.a16 ? (srow >> 4) : srow) * kgroups);
  const int voff_sb = (int)((p.b16 ? (srow >> 4) : srow) * kgroups);

  v4i32 sta[8], stb[8], ssa, ssb;   // one K step of this wave's share, in flight
  // part q (0..3) of step kb: code rows 2q and 2q+1 of both operands, scales with q = 3
  auto gload_part = [&](int kb, int q) {
#pragma unroll
    for (int i = 2 * q; i < 2 * q + 2; ++i) {
      const int off = voff_code + (int)__builtin_amdgcn_readfirstlane((uint32_t)(8 * i * rowb + (kbeg + kb) * kRowB2));
      sta[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
      stb[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
    }
    if (q == 3) {
      const int soff = (int)__builtin_amdgcn_readfirstlane((uint32_t)((kbeg + kb) * 16));
      ssa = __builtin_amdgcn_raw_buffer_load_b128(rsa, voff_sa + soff, 0, 0);
      ssb = __builtin_amdgcn_raw_buffer_load_b128(rsb, voff_sb + soff, 0, 0);
    }
  };
  auto gload = [&](int kb) {
#pragma unroll
    for (int q = 0; q < 4; ++q) gload_part(kb, q);
  };
  // the part of the staged step that gload_part(., q) loaded
  auto swrite_part = [&](int stage, int q) {
    uint8_t *base = lds + stage * kStageB2;
#pragma unroll
    for (int i = 2 * q; i < 2 * q + 2; ++i) {
      uint8_t *rowp = base + (8 * wave + i) * 1024 + ((i & 1) ? wr_o : wr_e);
      *reinterpret_cast<v4i32 *>(rowp) = sta[i];
      *reinterpret_cast<v4i32 *>(rowp + kCodesB2) = stb[i];
    }
    if (q == 3) {   // scales: dword j of row r to [j][r]
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        reinterpret_cast<int32_t *>(base + 2 * kCodesB2 + j * 1024)[srow] = ssa[j];
        reinterpret_cast<int32_t *>(base + 2 * kCodesB2 + kScalesB2 + j * 1024)[srow] = ssb[j];
      }
    }
  };
  auto swrite = [&](int stage) {
#pragma unroll
    for (int q = 0; q < 4; ++q) swrite_part(stage, q);
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Software pipeline.  Within a K step, the operands of MFMA sub-step s+1 are read
  // from LDS and dequantized while the 16 MFMAs of sub-step s run (scheduling barriers
  // interleave each MFMA with LDS accesses and a few VALU instructions).  Across K steps,
  // the stage barrier sits after the last LDS read of the current stage (sub-step 11): past it,
  // the loads of step kb+2 go into the freed stage and the first operands of step kb+1
  // are prepared under the last MFMAs of step kb.
  uint4 ca[2][4], cb[2][4];      // packed codes of two 32-element chunks (double buffer)
  uint32_t sra[2][4], srb[2][4]; // their scale dwords, as read
  half2_t hsa[2][4], hsb[2][4];  // their block scales
  half8_t ao[2][4], bo[2][4];    // dequantized operands of two sub-steps
  // chunk j of a stage: 16 code bytes per block row and the dword of scale bytes that holds
  // the two (K groups 4j + 2h, 4j + 2h + 1) covering them, into buffer j & 1; the scales
  // are converted by convert_scales a sub-step later, so that no instruction waits for
  // these LDS reads right after they are issued
  auto load_chunk16 = [&](const uint8_t *st, int j) {
    const int slot = ((2 * j + h) ^ ((l32 >> 1) & 7)) * 16;
    const uint8_t *ssa = st + 2 * kCodesB2, *ssb = ssa + kScalesB2;
    const int b = j & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ca[b][i] = lds16(st + (wm * 128 + i * 32 + l32) * kRowB2 + slot);
      cb[b][i] = lds16(st + kCodesB2 + (wn * 128 + i * 32 + l32) * kRowB2 + slot);
      sra[b][i] = *reinterpret_cast<const uint32_t *>(ssa + j * 1024 + (wm * 128 + i * 32 + l32) * 4);
      srb[b][i] = *reinterpret_cast<const uint32_t *>(ssb + j * 1024 + (wn * 128 + i * 32 + l32) * 4);
    }
  };
  auto convert_scales = [&](int b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hsa[b][i] = e4m3_pair_f16(sra[b][i], h);
      hsb[b][i] = e4m3_pair_f16(srb[b][i], h);
    }
  };
  auto dequant_step = [&](int s, half8_t (&ad)[4], half8_t (&bd)[4]) {
    const int q = s & 3, b = (s >> 2) & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t wa = q == 0 ? ca[b][i].x : q == 1 ? ca[b][i].y : q == 2 ? ca[b][i].z : ca[b][i].w;
      const uint32_t wb = q == 0 ? cb[b][i].x : q == 1 ? cb[b][i].y : q == 2 ? cb[b][i].z : cb[b][i].w;
      ad[i] = dequant8_f16(wa, hsa[b][i][q >> 1]);
      bd[i] = dequant8_f16(wb, hsb[b][i][q >> 1]);
    }
  };

  // Pipeline: chunk j of a K step is read from LDS four sub-steps before its first use;
  // the operands of sub-step s+1 are dequantized under the MFMAs of sub-step s.  The
  // stage barrier sits at sub-step 11, after the last LDS read of the current stage;
  // past it step kb+2 is written into the freed stage, chunk 0 of step kb+1 is read at
  // sub-step 12 and its first operands prepared at sub-step 15.
  gload(0);
  swrite(0);
  if (nk > 1) {
    gload(1);
    swrite(1);
  }
  if (nk > 2) gload(2);   // held in registers until stage 0 is free
  __syncthreads();
  load_chunk16(lds, 0);
  convert_scales(0);
  dequant_step(0, ao[0], bo[0]);
  for (int kb = 0; kb < nk; ++kb) {
    const uint8_t *st = lds + (kb & 1) * kStageB2;
    const uint8_t *st_next = lds + ((kb + 1) & 1) * kStageB2;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int cur = s & 1;
      if ((s & 3) == 0 && s < 12) load_chunk16(st, (s >> 2) + 1);
      // the chunk read one sub-step ago (at s = 12, chunk 0 of the next step): its scales
      if ((s & 3) == 1) convert_scales(((s >> 2) + 1) & 1);
      if (s == 11) __syncthreads();   // every wave is done with st; step kb+1's writes are visible
      // step kb+2 into the freed stage, one quarter per sub-step from 11 on; each quarter's
      // registers then take the same quarter of step kb+3
      if (s >= 11 && s < 15 && kb + 2 < nk) swrite_part(kb & 1, s - 11);
      if (s >= 12 && kb + 3 < nk) gload_part(kb + 3, s - 12);
      if (s == 12 && kb + 1 < nk) load_chunk16(st_next, 0);
      if (s + 1 < 16) dequant_step(s + 1, ao[cur ^ 1], bo[cur ^ 1]);
      else if (kb + 1 < nk) dequant_step(0, ao[0], bo[0]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ao[cur][i], bo[cur][jj], acc[i][jj], 0, 0, 0);
      // each MFMA followed by up to one LDS read, one LDS write and five VALU instructions
      // (LDS traffic threaded through the MFMAs rather than issued in a block: 1.25 -> 1.23
      // ms on workload 5)
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0); // one LDS write
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0); // up to five VALU
      }
    }
  }

  if (item >= 0) {
    // Split item: the partial tile goes to its slot as [wave][i][jj][r / 4][lane] groups of
    // four, then the item counts itself.  Slots are written and read by 128-bit buffer
    // accesses with the agent-scope cache policy (aux 16: the bits the compiler gives
    // agent-scope atomic loads and stores), which are coherent across the XCDs' L2 caches
    // by themselves, and the count is taken only after every store of the workgroup has
    // completed: no cache write-back or invalidation is needed, which would also flush the
    // L2 under the other workgroups of the XCD.  The last arrival sums all slots of the
    // tile in split order.
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(ws + kGemmCtrBytes, (int64_t)kGemmMaxItems * kT2 * kT2 * 4);
    const int tile = item / splits;
    constexpr int kSlotB = kT2 * kT2 * 4;   // bytes per slot
    const int lane_off = (wave * 16 * 4 * 64 + lane) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v4i32 v = {(int)__float_as_uint(acc[i][jj][4 * q]), (int)__float_as_uint(acc[i][jj][4 * q + 1]),
                     (int)__float_as_uint(acc[i][jj][4 * q + 2]), (int)__float_as_uint(acc[i][jj][4 * q + 3])};
          __builtin_amdgcn_raw_buffer_store_b128(v, rs, lane_off + ((i * 4 + jj) * 4 + q) * 64 * 16,
                                                 (int)__builtin_amdgcn_readfirstlane((uint32_t)(item * kSlotB)), 16);
        }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's stores have completed
    __syncthreads();
    if (tid == 0) {
      uint32_t *ctr = reinterpret_cast<uint32_t *>(ws) + tile;
      const uint32_t before = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = before == (uint32_t)splits - 1u;
      if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sk_last = last ? 1u : 0u;
    }
    __syncthreads();
    if (!sk_last) return;
    for (int sp = 0; sp < splits; ++sp) {
      const int soff = (int)__builtin_amdgcn_readfirstlane((uint32_t)((tile * splits + sp) * kSlotB));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const v4i32 v = __builtin_amdgcn_raw_buffer_load_b128(rs, lane_off + ((i * 4 + jj) * 4 + q) * 64 * 16, soff, 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float f = __uint_as_float((uint32_t)v[e]);
              acc[i][jj][4 * q + e] = sp == 0 ? f : acc[i][jj][4 * q + e] + f;
            }
          }
    }
  }

  // Epilogue.  Accumulator element r of block (i, jj) sits at row 32 i + 8 (r / 4) + 4 h +
  // r % 4 and column 32 jj + l32 of the wave's 128 x 128 block.  A tile wholly inside C
  // takes the unchecked path: one row address per (i, r), the four column blocks as
  // immediate offsets, bf16 by the hardware conversion (nearest-even; checked on every
  // binary32 against the rounding of the guarded path below), non-temporal stores (C is
  // written once; keeping it out of the caches leaves them to the operands, 2-5 % here).
  const float alpha = (*p.ag) * (*p.bg);
  const int rbase = m0 + wm * 128 + 4 * h, cbase = n0 + wn * 128 + l32;
  if (m0 + kT2 <= p.M && n0 + kT2 <= p.N) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t off = (int64_t)(rbase + i * 32 + 8 * (r >> 2) + (r & 3)) * p.ldc + cbase;
        if (F32) {
          float *dst = reinterpret_cast<float *>(p.c) + off;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) __builtin_nontemporal_store(acc[i][jj][r] * alpha, dst + jj * 32);
        } else {
          uint16_t *dst = reinterpret_cast<uint16_t *>(p.c) + off;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            __builtin_nontemporal_store(bf16_bits_rn(acc[i][jj][r] * alpha), dst + jj * 32);
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rbase + i * 32 + 8 * (r >> 2) + (r & 3);
        const int col = cbase + jj * 32;
        if (row < p.M && col < p.N) {
          const float v = acc[i][jj][r] * alpha;
          if (F32) {
            reinterpret_cast<float *>(p.c)[(int64_t)row * p.ldc + col] = v;
          } else {
            const uint32_t u = __float_as_uint(v);
            const uint32_t bb = ((u & 0x7FFFFFFFu) > 0x7F800000u) ? ((u >> 16) | 0x40u)
                                                                 : ((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
            reinterpret_cast<uint16_t *>(p.c)[(int64_t)row * p.ldc + col] = (uint16_t)bb;
          }
        }
      }
}

constexpr int kMinSplitSteps = 8;

// Compute units of the current device (cached per device; a racing writer stores the
// same value).
int cu_count() {
  static int cache[64] = {};
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64 && cache[dev]) return cache[dev];
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  if (dev >= 0 && dev < 64) cache[dev] = cus;
  return cus;
}

}  // namespace

hipError_t launch_gemm(const GemmLaunch &g, hipStream_t stream) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  GemmParams p;
  p.ac = g.a.codes; p.as = g.a.scales; p.ag = g.a.global_dec; p.a16 = g.a.blocking;
  p.bc = g.b.codes; p.bs = g.b.scales; p.bg = g.b.global_dec; p.b16 = g.b.blocking;
  p.M = (int)g.M; p.N = (int)g.N; p.K = (int)g.K; p.ldc = g.ldc; p.c = g.c;
  if (g.K > 0 && g.K % 256 == 0) {
    const int tm = (int)((g.M + kT2 - 1) / kT2), tn = (int)((g.N + kT2 - 1) / kT2);
    const int tiles = tm * tn, nk = (int)(g.K / 256);
    // One workgroup per CU: split the tiles of a last, partial round along K so that it
    // keeps every CU busy.  A split item moves 256 KB of partial tile out and its tile's
    // last item moves all of them back in, about the time of a few K steps, so each item
    // keeps at least kMinSplitSteps K steps (at most 8 splits).
    int t_dp = tiles, splits = 1;
    if (g.ws) {
      const int cus = cu_count();
      const int rest = tiles % cus;
      if (rest > 0) {
        int sp = min(min(cus, kGemmMaxItems) / rest, min(8, nk / kMinSplitSteps));
        if (sp >= 2) {
          t_dp = tiles - rest;
          splits = sp;
        }
      }
    }
    const unsigned grid = (unsigned)(t_dp + (tiles - t_dp) * splits);
    uint8_t *ws = static_cast<uint8_t *>(g.ws);
    if (g.out_f32) gemm256_kernel<true><<<grid, 256, 0, stream>>>(p, tm, tn, t_dp, splits, ws);
    else gemm256_kernel<false><<<grid, 256, 0, stream>>>(p, tm, tn, t_dp, splits, ws);
    return hipGetLastError();
  }
  const int tiles_n = (int)((g.N + kBN - 1) / kBN);
  const unsigned grid = (unsigned)(tiles_n * ((g.M + kBM - 1) / kBM));
  const bool k32 = (g.K % 32) == 0;
  if (g.out_f32) {
    if (k32) gemm_kernel<true, true><<<grid, 256, 0, stream>>>(p, tiles_n);
    else gemm_kernel<true, false><<<grid, 256, 0, stream>>>(p, tiles_n);
  } else {
    if (k32) gemm_kernel<false, true><<<grid, 256, 0, stream>>>(p, tiles_n);
    else gemm_kernel<false, false><<<grid, 256, 0, stream>>>(p, tiles_n);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
