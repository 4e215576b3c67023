// mxfp4.hip -- MXFP4 quantize, dequantize and GEMM on gfx950.
//
// MXFP4 is the format the pages set NVFP4 against: 32-element blocks sharing one
// power-of-two (E8M0) scale, no tensor scale (NVIDIA developer blog zh-cn "NVFP4 trains with
// precision of 16-bit and speed and efficiency of 4-bit", section "用于预训练的 NVFP4
// 量化配方", first two bullets; prism.simon-ai.net article 7890, section "MVFP4与MXFP4：
// 通过缩放实现低精度推理").  The pages fix the block size and the scale type, not how the
// power of two is chosen; the rule here is the one of the OCP Microscaling Formats v1.0
// specification: X = 2^(floor(log2 amax) - 2), 2 being the exponent of E2M1's largest
// value (6 = 1.5 * 2^2), clamped to E8M0's range; a block holding inf or NaN gets the NaN
// scale 0xFF and zero codes.  Elements are v / X rounded to nearest-even E2M1 (saturating
// at 6).
//
// gfx950's scaled matrix instructions take this format as it is: the GEMM feeds packed
// codes and scale bytes straight to v_mfma_scale_f32_32x32x64_f8f6f4, with no
// dequantization.
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace {

// ---------------------------------------------------------------- quantize
// One lane per 8 elements (one 16-byte load, one dword of codes); the four lanes of a
// DPP quad hold one 32-element block and agree on its scale through two quad
// permutations.  Each lane handles kQU such pieces per pass, loads first.
constexpr int kQT = 256, kQU = 4;

template <bool CONTIG>
__global__ __launch_bounds__(kQT) void mx_quant_kernel(const uint16_t *__restrict__ x,
                                                       int64_t ld, uint32_t c8, uint32_t nchunks,
                                                       uint32_t *__restrict__ codes,
                                                       uint8_t *__restrict__ scales) {
  const uint32_t tid = threadIdx.x;
  for (uint32_t base = blockIdx.x * (kQT * kQU); base < nchunks; base += gridDim.x * (kQT * kQU)) {
    uint4 v[kQU];
#pragma unroll
    for (int u = 0; u < kQU; ++u) {
      const uint32_t idx = base + u * kQT + tid;
      v[u] = make_uint4(0u, 0u, 0u, 0u);
      if (idx < nchunks) {
        const uint16_t *p;
        if (CONTIG) {
          p = x + (uint64_t)idx * 8u;
        } else {
          const uint32_t r = idx / c8;
          p = x + (int64_t)r * ld + (uint64_t)(idx - r * c8) * 8u;
        }
        v[u] = *reinterpret_cast<const uint4 *>(p);
      }
    }
#pragma unroll
    for (int u = 0; u < kQU; ++u) {
      const uint32_t idx = base + u * kQT + tid;
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      // |x| as bf16 bits orders like the magnitudes; inf and NaN have the top exponent
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
      m = max(m, lane_xor1(m));
      m = max(m, lane_xor2(m));
      // floor(log2 amax) = E - 127 for the biased exponent E of a normal amax, so the
      // biased scale is E - 2; subnormal and zero blocks clamp to 0 (2^-127)
      const uint32_t e = m >> 7;
      const bool bad = e == 0xFFu;
      const uint32_t sbyte = bad ? 0xFFu : (e > 2u ? e - 2u : 0u);
      // 1 / X = 2^(127 - sbyte), a normal binary32 for sbyte <= 252 (the largest a finite
      // bf16 block reaches); v * (1 / X) rounds once, like the exact quotient would
      const float rr = __uint_as_float((254u - min(sbyte, 252u)) << 23);
      uint32_t c = 0;
      c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, bf16_lo(w[0]) * rr, bf16_hi(w[0]) * rr, 1.0f, 0);
      c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, bf16_lo(w[1]) * rr, bf16_hi(w[1]) * rr, 1.0f, 1);
      c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, bf16_lo(w[2]) * rr, bf16_hi(w[2]) * rr, 1.0f, 2);
      c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, bf16_lo(w[3]) * rr, bf16_hi(w[3]) * rr, 1.0f, 3);
      if (bad) c = 0u;
      if (idx < nchunks) {
        codes[idx] = c;
        if ((tid & 3u) == 0u) scales[idx >> 2] = (uint8_t)sbyte;
      }
    }
  }
}

// ---------------------------------------------------------------- dequantize
// y = e2m1(code) * 2^(s - 127), exact in binary32 (at most two significant bits, and the
// smallest value 2^-128 is a binary32 subnormal); NaN for s = 0xFF.  The values are also
// exact in bf16, so the bf16 output is the top half of the binary32 pattern.
template <int B>
__device__ __forceinline__ void mx_decode_byte(uint32_t c, int e, float *v) {
  const float2_t f = e2m1_decode_pair<B>(c);   // exact
  v[2 * B] = __builtin_ldexpf(f[0], e);
  v[2 * B + 1] = __builtin_ldexpf(f[1], e);
}

// One thread per 16 bytes of output: 8 elements for bf16, 4 for fp32 (4 or 2 code bytes),
// so each store instruction of a wave writes 1 KiB of consecutive output; non-temporal
// stores (the output is written once).  Part q covers elements E q .. E q + E - 1 of the
// row-major element order, whose 32-element block is (E q) / 32.
template <bool F32, bool CONTIG>
__global__ __launch_bounds__(256) void mx_dequant_kernel(const uint8_t *__restrict__ codes,
                                                         const uint8_t *__restrict__ scales,
                                                         uint32_t cparts, uint64_t nparts,
                                                         int64_t ld, void *__restrict__ y) {
  typedef int v4i32 __attribute__((ext_vector_type(4)));
  constexpr uint32_t E = F32 ? 4 : 8;
  for (uint64_t q = (uint64_t)blockIdx.x * 256u + threadIdx.x; q < nparts;
       q += (uint64_t)gridDim.x * 256u) {
    const uint32_t c = F32 ? (uint32_t)reinterpret_cast<const uint16_t *>(codes)[q]
                           : reinterpret_cast<const uint32_t *>(codes)[q];
    const uint32_t s = scales[(q * E) >> 5];
    const int e = (int)s - 127;
    float v[8];
    mx_decode_byte<0>(c, e, v);
    mx_decode_byte<1>(c, e, v);
    if (!F32) {
      mx_decode_byte<2>(c, e, v);
      mx_decode_byte<3>(c, e, v);
    }
    if (s == 0xFFu) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = __builtin_nanf("");
    }
    uint64_t off;
    if (CONTIG) {
      off = q * E;
    } else {
      const uint64_t r = q / cparts;
      off = r * (uint64_t)ld + (q - r * cparts) * E;
    }
    v4i32 w;
    if (F32) {
      w = (v4i32){(int)__float_as_uint(v[0]), (int)__float_as_uint(v[1]),
                  (int)__float_as_uint(v[2]), (int)__float_as_uint(v[3])};
      __builtin_nontemporal_store(w, reinterpret_cast<v4i32 *>(reinterpret_cast<float *>(y) + off));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (int)((__float_as_uint(v[2 * i]) >> 16) | (__float_as_uint(v[2 * i + 1]) & 0xFFFF0000u));
      __builtin_nontemporal_store(w, reinterpret_cast<v4i32 *>(reinterpret_cast<uint16_t *>(y) + off));
    }
  }
}

// ---------------------------------------------------------------- GEMM
// C = A . B^T, A: M x K and B: N x K MXFP4 (K contiguous).
//
// One 256-thread workgroup per CU computes a 256 x 256 tile; each wave owns 128 x 128
// (4 x 4 blocks of 32 x 32, 256 fp32 accumulators).  K advances 256 elements per step:
// every row of A and B brings one 128-byte line of codes and 8 scale bytes, which travel
// through registers into one of two LDS stages while the waves compute on the other.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands FP4 covers K = 64: lane (l32, h)
// gives row l32 of its block, K elements 32h .. 32h+31 as 16 packed bytes (element j at
// nibble j, low nibble first: the storage order of the codes), and in a scale register
// the E8M0 byte of exactly that 32-element block.  MFMA sub-step s of a K step takes
// 32-element chunk 2s + h, so a lane needs scale bytes h, h+2, h+4, h+6 of its row over the
// step: after the LDS read of the row's 8 bytes one byte permute gathers them into one
// register, and sub-step s selects byte s with the instruction's operand byte select.  The accumulator layout is that of the f16 32x32
// MFMA: element r of lane (l32, h) is row 8 (r / 4) + 4 h + r % 4, column l32.
//
// LDS: codes of a row at slot chunk ^ ((row >> 1) & 7), 16 bytes each, so the 128-bit
// reads of 16 consecutive rows cover the 64 banks once; scales as [row][8 bytes].
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef int v4i32 __attribute__((ext_vector_type(4)));
typedef int v8i32 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kMT = 256;                  // tile rows and columns
constexpr int kMRowB = 128;               // code bytes per row per K step
constexpr int kMCodesB = kMT * kMRowB;    // 32 KB per operand per stage
constexpr int kMScalesB = 2 * kMT * 4;    // 2 KB per operand per stage
constexpr int kMStageB = 2 * kMCodesB + 2 * kMScalesB;

struct MxGemmParams {
  const uint8_t *ac, *as, *bc, *bs;
  int M, N, K;
  int64_t ldc;
  void *c;
};

__device__ __forceinline__ v8i32 widen(v4i32 a) {
  // FP4 operands occupy the first four registers of the 8-register operand
  return __builtin_shufflevector(a, (v4i32){0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
}

// MFMA blocks (i, j) for i in [I0, I1) of sub-step S (operand byte select S: scale byte
// h + 2 S of the row, see the LDS layout of the scales)
template <int S, int I0, int I1>
__device__ __forceinline__ void mx_mfma(floatx16 (&acc)[4][4], const v4i32 (&a)[4],
                                        const v4i32 (&b)[4], const uint32_t (&sa)[4],
                                        const uint32_t (&sb)[4]) {
#pragma unroll
  for (int i = I0; i < I1; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          widen(a[i]), widen(b[j]), acc[i][j], 4, 4, S, (int)sa[i], S, (int)sb[j]);
}

// Instruction-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008, kSgVmemRead = 0x020, kSgDsRead = 0x100, kSgDsWrite = 0x200;

// One 256 x 256 output tile (index `tile`) by the calling workgroup.
template <bool F32, bool KFULL>
__device__ __forceinline__ void mx_tile(const MxGemmParams &p, int tile, int tiles_m, int tiles_n,
                                        uint8_t *lds) {
  // tile order: the tiles whose index is congruent mod 8 (the workgroups of one XCD, which
  // takes every eighth block) form a contiguous range, walked four tile-rows at a time
  // so concurrent tiles share A and B
  const int G = tiles_m * tiles_n;
  int bid = tile;
  if ((G & 7) == 0) bid = (bid & 7) * (G >> 3) + (bid >> 3);
  const int gm = 4;
  const int band = bid / (gm * tiles_n), in_band = bid - band * gm * tiles_n;
  const int rows_in_band = min(gm, tiles_m - band * gm);
  const int tm = band * gm + in_band % rows_in_band;
  const int tn = in_band / rows_in_band;
  const int m0 = tm * kMT, n0 = tn * kMT;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, l32 = lane & 31;
  const int rowb = p.K >> 1;        // code bytes per row
  const int sgr = p.K >> 5;         // scale bytes (32-element chunks) per row
  const int nk = (p.K + 255) >> 8;  // K steps; the last may be partial

  // Buffer resources start at the tile's first row and end at the operand's last, so a
  // row past M or N reads zero codes and zero scale bytes and adds nothing.
  const int ra_rows = min(p.M - m0, kMT), rb_rows = min(p.N - n0, kMT);
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(p.ac + (int64_t)m0 * rowb, (int64_t)ra_rows * rowb);
  const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(p.bc + (int64_t)n0 * rowb, (int64_t)rb_rows * rowb);
  const __amdgpu_buffer_rsrc_t rsa = buffer_rsrc(p.as + (int64_t)m0 * sgr, (int64_t)ra_rows * sgr);
  const __amdgpu_buffer_rsrc_t rsb = buffer_rsrc(p.bs + (int64_t)n0 * sgr, (int64_t)rb_rows * sgr);
  const __amdgpu_buffer_rsrc_t r0 = buffer_rsrc(p.ac, 0);

  // Load i (0..7) of wave w brings tile row 64 w + 8 i + lane / 8, chunk lane % 8, which
  // goes to slot chunk ^ ((row >> 1) & 7) = chunk ^ (4 (i & 1) + lane / 16).  Scales: lane
  // l of wave w brings the 8 bytes of tile row 64 w + l.
  const int voff_code = (64 * wave + (lane >> 3)) * rowb + (lane & 7) * 16;
  const int wr_e = (lane >> 3) * kMRowB + (((lane & 7) ^ (lane >> 4)) * 16);
  const int wr_o = (lane >> 3) * kMRowB + (((lane & 7) ^ (4 + (lane >> 4))) * 16);
  const int srow = 64 * wave + lane;
  const int voff_s = srow * sgr;

  // One K step of this wave's share in registers: code rows 8 i + lane / 8 (i = 0..7) of
  // both operands and the scale bytes of row lane.
  struct Staged {
    v4i32 a[8], b[8];
    v2i32 sa, sb;
  };
  // part q (0..3) of step kb into `g`: code rows 8 i + lane / 8 for i = 2q, 2q + 1 of
  // both operands, and with q = 3 the scale bytes.  With live == false every load goes
  // through an empty resource and returns zero without touching memory.
  auto gload_part = [&](Staged &g, int kb, int q, bool live) {
    const __amdgpu_buffer_rsrc_t ga = live ? ra : r0, gb = live ? rb : r0;
    // chunks past K (only in a partial last step) read as zero codes and zero scales
    const int valid = KFULL ? 8 : min(8, sgr - 8 * kb);
#pragma unroll
    for (int i = 2 * q; i < 2 * q + 2; ++i) {
      // the whole offset in the per-lane offset, which the range check covers
      const int off = voff_code + (int)__builtin_amdgcn_readfirstlane((uint32_t)(8 * i * rowb + kb * kMRowB));
      g.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ga, off, 0, 0);
      g.b[i] = __builtin_amdgcn_raw_buffer_load_b128(gb, off, 0, 0);
      if (!KFULL && (lane & 7) >= valid) {
        g.a[i] = (v4i32){0, 0, 0, 0};
        g.b[i] = (v4i32){0, 0, 0, 0};
      }
    }
    if (q != 3) return;
    const __amdgpu_buffer_rsrc_t gsa = live ? rsa : r0, gsb = live ? rsb : r0;
    if (KFULL) {
      const int soff = (int)__builtin_amdgcn_readfirstlane((uint32_t)(kb * 8));
      g.sa = __builtin_amdgcn_raw_buffer_load_b64(gsa, voff_s + soff, 0, 0);
      g.sb = __builtin_amdgcn_raw_buffer_load_b64(gsb, voff_s + soff, 0, 0);
    } else {
      // the scale rows of a K that is not a multiple of 256 are not 8-byte aligned
      uint32_t a2[2] = {0u, 0u}, b2[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < valid) {
          const uint32_t av = __builtin_amdgcn_raw_buffer_load_b8(gsa, voff_s + 8 * kb + j, 0, 0);
          const uint32_t bv = __builtin_amdgcn_raw_buffer_load_b8(gsb, voff_s + 8 * kb + j, 0, 0);
          a2[j >> 2] |= av << (8 * (j & 3));
          b2[j >> 2] |= bv << (8 * (j & 3));
        }
      }
      g.sa = (v2i32){(int)a2[0], (int)a2[1]};
      g.sb = (v2i32){(int)b2[0], (int)b2[1]};
    }
  };
  auto gload = [&](Staged &g, int kb, bool live) {
#pragma unroll
    for (int q = 0; q < 4; ++q) gload_part(g, kb, q, live);
  };
  auto swrite = [&](const Staged &g, int stage) {
    uint8_t *base = lds + stage * kMStageB;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint8_t *rowp = base + (8 * wave + i) * 1024 + ((i & 1) ? wr_o : wr_e);
      *reinterpret_cast<v4i32 *>(rowp) = g.a[i];
      *reinterpret_cast<v4i32 *>(rowp + kMCodesB) = g.b[i];
    }
    // the 8 scale bytes of row srow, as they are
    *reinterpret_cast<v2i32 *>(base + 2 * kMCodesB + srow * 8) = g.sa;
    *reinterpret_cast<v2i32 *>(base + 2 * kMCodesB + kMScalesB + srow * 8) = g.sb;
  };
  // a lane's scale word for the step: bytes h, h+2, h+4, h+6 of its row (sub-step s
  // selects byte s)
  const uint32_t sel_h = h ? 0x07050301u : 0x06040200u;
  auto read_scales = [&](const uint8_t *st, uint32_t (&sa)[4], uint32_t (&sb)[4]) {
    const uint8_t *sp = st + 2 * kMCodesB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v2i32 da = *reinterpret_cast<const v2i32 *>(sp + (wm * 128 + i * 32 + l32) * 8);
      const v2i32 db = *reinterpret_cast<const v2i32 *>(sp + kMScalesB + (wn * 128 + i * 32 + l32) * 8);
      sa[i] = __builtin_amdgcn_perm((uint32_t)da[1], (uint32_t)da[0], sel_h);
      sb[i] = __builtin_amdgcn_perm((uint32_t)db[1], (uint32_t)db[0], sel_h);
    }
  };
  // operands of sub-step s, in the order the MFMAs (i-major) first need them
  auto read_ops = [&](const uint8_t *st, int s, v4i32 (&a)[4], v4i32 (&b)[4]) {
    const int slot = ((2 * s + h) ^ ((l32 >> 1) & 7)) * 16;
    const uint8_t *pa = st + (wm * 128 + l32) * kMRowB + slot;
    const uint8_t *pb = st + kMCodesB + (wn * 128 + l32) * kMRowB + slot;
    a[0] = *reinterpret_cast<const v4i32 *>(pa);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const v4i32 *>(pb + j * 32 * kMRowB);
#pragma unroll
    for (int i = 1; i < 4; ++i) a[i] = *reinterpret_cast<const v4i32 *>(pa + i * 32 * kMRowB);
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Pipeline.  The operands of sub-step s + 1 are read from LDS under the MFMAs of
  // sub-step s, one read after every second MFMA: with one wave per SIMD an instruction
  // behind a waiting MFMA cannot issue, so the memory work is threaded between them.  The
  // stage barrier follows the last LDS read of the current stage (sub-step 3's operands,
  // read under sub-step 2's first half); past it, step kb + 2 goes from its staging
  // registers into the freed stage under sub-step 2's second half.  Two register sets
  // alternate: the set just written takes the first half of step kb + 4 under sub-step 3
  // and its second half under sub-steps 0 and 1 of the next step, so the vector memory
  // instructions are spread over the whole step rather than queued behind one group of
  // MFMAs, and every load has more than a K step to arrive.  (A K that is not a multiple
  // of 256 uses one set and loads step kb + 3 whole under sub-step 3: its byte-wise scale
  // loads need the registers, and such shapes are small.)  Each step is one basic block:
  // past the last steps the writes go to a stage no one reads again, the loads go through
  // an empty buffer resource, and the reads fetch stale words no one uses.
  Staged g0, g1;
  Staged &g_odd = KFULL ? g1 : g0;
  gload(g0, 0, nk > 0);
  swrite(g0, 0);
  gload(g0, 1, nk > 1);
  swrite(g0, 1);
  gload(g0, 2, nk > 2);
  if (KFULL) {
    gload_part(g1, 3, 0, nk > 3);
    gload_part(g1, 3, 1, nk > 3);
  }
  __syncthreads();
  v4i32 a0[4], b0[4], a1[4], b1[4];
  uint32_t sa[4], sb[4];
  read_scales(lds, sa, sb);
  read_ops(lds, 0, a0, b0);
  // step kb: `cur` holds step kb + 2 (written here, then reloaded), `oth` receives the
  // second half of step kb + 3
  auto kstep = [&](int kb, Staged &cur, Staged &oth) __attribute__((always_inline)) {
    const uint8_t *st = lds + (kb & 1) * kMStageB;
    const uint8_t *stn = lds + ((kb + 1) & 1) * kMStageB;
    if (KFULL) {
      gload_part(oth, kb + 3, 2, kb + 3 < nk);
      gload_part(oth, kb + 3, 3, kb + 3 < nk);
    }
    read_ops(st, 1, a1, b1);
    mx_mfma<0, 0, 4>(acc, a0, b0, sa, sb);
    read_ops(st, 2, a0, b0);
    mx_mfma<1, 0, 4>(acc, a1, b1, sa, sb);
    v4i32 a2[4], b2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a2[i] = a0[i];
      b2[i] = b0[i];
    }
    read_ops(st, 3, a1, b1);
    mx_mfma<2, 0, 2>(acc, a2, b2, sa, sb);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgVmemRead, 1, 0);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
    }
    __syncthreads();   // every wave is done with st; step kb + 1's stage is visible
    swrite(cur, kb & 1);
    mx_mfma<2, 2, 4>(acc, a2, b2, sa, sb);
    if (KFULL) {
      gload_part(cur, kb + 4, 0, kb + 4 < nk);
      gload_part(cur, kb + 4, 1, kb + 4 < nk);
    } else {
      gload(cur, kb + 3, kb + 3 < nk);
    }
    uint32_t san[4], sbn[4];
    read_scales(stn, san, sbn);
    read_ops(stn, 0, a0, b0);
    mx_mfma<3, 0, 4>(acc, a1, b1, sa, sb);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgDsWrite, 3, 0);
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgVmemRead, KFULL ? 1 : 2, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] = san[i];
      sb[i] = sbn[i];
    }
  };
  int kb = 0;
  for (; kb + 1 < nk; kb += 2) {
    kstep(kb, g0, g_odd);
    kstep(kb + 1, g_odd, g0);
  }
  if (kb < nk) kstep(kb, g0, g_odd);

  // Epilogue: element r of block (i, jj) is row 32 i + 8 (r / 4) + 4 h + r % 4, column
  // 32 jj + l32 of the wave's 128 x 128 block.  bf16 output rounds to nearest-even.
  const int rbase = m0 + wm * 128 + 4 * h, cbase = n0 + wn * 128 + l32;
  const bool full = m0 + kMT <= p.M && n0 + kMT <= p.N;
  if (!F32 && full && (p.ldc & 7) == 0) {
    // bf16 through LDS: each wave stages its 128 x 128 block row-major (rows padded to
    // 272 bytes, so the two lane halves, 4 rows apart, hit disjoint banks), then writes
    // it back with one 16-byte store per lane per 4 rows: 32 stores instead of 256
    // two-byte ones.  The stores are non-temporal: C is written once and never read
    // here, and keeping it out of the caches leaves them to the operands (measured
    // ~10 % faster on the workload-5 product).
    constexpr int kOutStride = 272;
    __syncthreads();   // every wave is done with the stages
    uint8_t *ob = lds + wave * (128 * kOutStride);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          *reinterpret_cast<uint16_t *>(ob + row * kOutStride + (jj * 32 + l32) * 2) =
              bf16_bits_rn(acc[i][jj][r]);
        }
    const int crow = lane >> 4, cchunk = lane & 15;
    uint16_t *cdst = reinterpret_cast<uint16_t *>(p.c) + (int64_t)(m0 + wm * 128 + crow) * p.ldc +
                     n0 + wn * 128 + cchunk * 8;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const v4i32 v = *reinterpret_cast<const v4i32 *>(ob + (4 * t + crow) * kOutStride + cchunk * 16);
      __builtin_nontemporal_store(v, reinterpret_cast<v4i32 *>(cdst + (int64_t)(4 * t) * p.ldc));
    }
    return;
  }
  if (full) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t off = (int64_t)(rbase + i * 32 + 8 * (r >> 2) + (r & 3)) * p.ldc + cbase;
        if (F32) {
          float *dst = reinterpret_cast<float *>(p.c) + off;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) __builtin_nontemporal_store(acc[i][jj][r], dst + jj * 32);
        } else {
          uint16_t *dst = reinterpret_cast<uint16_t *>(p.c) + off;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) dst[jj * 32] = bf16_bits_rn(acc[i][jj][r]);
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
          const int64_t off = (int64_t)row * p.ldc + col;
          if (F32) reinterpret_cast<float *>(p.c)[off] = acc[i][jj][r];
          else reinterpret_cast<uint16_t *>(p.c)[off] = bf16_bits_rn(acc[i][jj][r]);
        }
      }
}

template <bool F32, bool KFULL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void mx_gemm_kernel(MxGemmParams p, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kMStageB];
  mx_tile<F32, KFULL>(p, blockIdx.x, tiles_m, tiles_n, lds);
}

uint32_t capped_grid(uint64_t items, uint32_t per_block, uint32_t cap) {
  const uint64_t g = (items + per_block - 1) / per_block;
  return (uint32_t)(g < cap ? g : cap);
}

}  // namespace

hipError_t launch_mx_quantize(const MxQuantLaunch &q, hipStream_t stream) {
  const uint64_t nchunks = (uint64_t)q.rows * (uint64_t)(q.cols / 8);
  if (nchunks == 0) return hipSuccess;
  const uint32_t grid = capped_grid(nchunks, kQT * kQU, 1u << 16);
  const bool contig = q.ld == q.cols;
  if (contig)
    mx_quant_kernel<true><<<grid, kQT, 0, stream>>>(q.x, q.ld, (uint32_t)(q.cols / 8), (uint32_t)nchunks,
                                                    reinterpret_cast<uint32_t *>(q.codes), q.scales);
  else
    mx_quant_kernel<false><<<grid, kQT, 0, stream>>>(q.x, q.ld, (uint32_t)(q.cols / 8), (uint32_t)nchunks,
                                                     reinterpret_cast<uint32_t *>(q.codes), q.scales);
  return hipGetLastError();
}

hipError_t launch_mx_dequantize(const MxDequantLaunch &d, hipStream_t stream) {
  const uint32_t e = d.out_f32 ? 4u : 8u;
  const uint64_t nparts = (uint64_t)d.rows * (uint64_t)(d.cols / e);
  if (nparts == 0) return hipSuccess;
  const uint32_t grid = capped_grid(nparts, 256, 16384);
  const uint32_t cparts = (uint32_t)(d.cols / e);
  const bool contig = d.ld_y == d.cols;
#define MX_DQ(F, C) mx_dequant_kernel<F, C><<<grid, 256, 0, stream>>>(d.codes, d.scales, cparts, nparts, d.ld_y, d.y)
  if (d.out_f32) { if (contig) MX_DQ(true, true); else MX_DQ(true, false); }
  else { if (contig) MX_DQ(false, true); else MX_DQ(false, false); }
#undef MX_DQ
  return hipGetLastError();
}

hipError_t launch_mx_gemm(const MxGemmLaunch &g, hipStream_t stream) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  MxGemmParams p;
  p.ac = g.a_codes; p.as = g.a_scales; p.bc = g.b_codes; p.bs = g.b_scales;
  p.M = (int)g.M; p.N = (int)g.N; p.K = (int)g.K; p.ldc = g.ldc; p.c = g.c;
  const int tm = (int)((g.M + kMT - 1) / kMT), tn = (int)((g.N + kMT - 1) / kMT);
  const bool kfull = g.K % 256 == 0;
  const int grid = tm * tn;
#define MX_GEMM(F, KF) mx_gemm_kernel<F, KF><<<grid, 256, 0, stream>>>(p, tm, tn)
  if (g.out_f32) { if (kfull) MX_GEMM(true, true); else MX_GEMM(true, false); }
  else { if (kfull) MX_GEMM(false, true); else MX_GEMM(false, false); }
#undef MX_GEMM
  return hipGetLastError();
}

}  // namespace nvfp4
