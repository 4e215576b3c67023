// nvfp4_device.hpp -- device-side building blocks of the NVFP4 kernels (gfx950).
//
// Everything here is binary32 with round-to-nearest-even and is built with
// -ffp-contract=off and without packed-FP32 instructions, so the results match a plain
// IEEE evaluation in the same operation order bit for bit.  Division is the compiler's
// correctly rounded fp32 division.
//
// Format sources: NVIDIA developer blog (zh-cn) "NVFP4 trains with precision of 16-bit
// and speed and efficiency of 4-bit", section "用于预训练的 NVFP4 量化配方" (bullets:
// 16-element micro-blocks, E4M3 scales, Hadamard transform, 2D blocks, stochastic
// rounding); prism.simon-ai.net article 7890, section "MVFP4格式的核心架构革新" (FP32 tensor
// scale above the E4M3 block scales).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr float kE2M1Max = 6.0f;
constexpr float kE4M3Max = 448.0f;
constexpr float kTensorRange = 2688.0f;  // 6 * 448: top of both formats
constexpr float kFltMax = 3.40282347e38f;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Unpack 16 bf16 values (two 16-byte words) to fp32 (exact), times the signs d of the
// transform given as a 16-bit mask (bit j set: d_j = -1; 0 for no transform).  A sign flip
// is an XOR of bit 31, which for the low bf16 of a word is the same as adding it after the
// shift, (w << 16) + s, and for the high one an AND-XOR, (w & 0xFFFF0000) ^ s: one
// instruction per value either way.
__device__ __forceinline__ void unpack16(const uint4 &a, const uint4 &b, float v[16],
                                         uint32_t signmask = 0u) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t s0 = ((signmask >> (2 * i)) & 1u) << 31;
    const uint32_t s1 = ((signmask >> (2 * i + 1)) & 1u) << 31;
    v[2 * i] = __uint_as_float((w[i] << 16) + s0);
    v[2 * i + 1] = __uint_as_float((w[i] & 0xFFFF0000u) ^ s1);
  }
}

// ---------------------------------------------------------------- RHT-16
// y = 1/4 * H16 * diag(d) * x, Sylvester H16.  Fixed evaluation order: sign flips (exact,
// done by unpack16), butterfly stages h = 1, 2, 4, 8 with (t_i, t_i+h) <- (t_i + t_i+h,
// t_i - t_i+h), then * 0.25 (which the callers fold into the block multiplier when exact).
__device__ __forceinline__ void rht16_stage(float v[16], int h) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i & h) continue;
    const float a = v[i], b = v[i + h];
    v[i] = a + b;
    v[i + h] = a - b;
  }
}

// t = H16 * d x from the signed values d x (before the final quarter).
__device__ __forceinline__ void rht16_unscaled(float v[16]) {
  rht16_stage(v, 1);
  rht16_stage(v, 2);
  rht16_stage(v, 4);
  rht16_stage(v, 8);
}

// Largest |t_i| of t = H16 * d x (from the signed values d x) as binary32 bits, without
// forming the last
// stage: for its pair (a, b), max(|a + b|, |a - b|) = |a| + |b| exactly, and rounding to
// nearest is monotonic and sign-symmetric, so the larger of the two rounded magnitudes is
// the rounded |a| + |b|.  Non-finite inputs give a result >= 0x7F800000.
__device__ __forceinline__ uint32_t rht16_absmax_bits(float v[16]) {
  rht16_stage(v, 1);
  rht16_stage(v, 2);
  rht16_stage(v, 4);
  uint32_t m = 0u;   // integer max of the bit patterns: a NaN is kept, not dropped
#pragma unroll
  for (int i = 0; i < 8; ++i)
    m = max(m, __float_as_uint(fabsf(v[i]) + fabsf(v[i + 8])) & 0x7FFFFFFFu);
  return m;
}

// ---------------------------------------------------------------- E4M3
// Nearest-even E4M3FN code of s >= 0, saturating to 448 (code 0x7E).  The hardware
// conversion rounds to nearest-even over the normal and subnormal E4M3 grid; clamping at
// 448 first gives the saturation (values from 464 up would otherwise become NaN).
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(s, kE4M3Max), 0.0f, 0, false) & 0xFFu;
}

// Value of an E4M3FN code (exact).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
}

// a / 6 rounded to nearest-even.  q0 = a * RN(1/6) is within an ulp; the residual
// a - 6 q0 is exact under FMA, and one correction step q0 + residual * RN(1/6) lands on
// the correctly rounded quotient for every binary32 a >= 2^-125 (an exhaustive property
// of binary32; the CPU tests check it).  Smaller a, where the residual is no longer
// exact, take the division.
__device__ __forceinline__ float div6(float a) {
  if (__float_as_uint(a) < 0x01000000u) return a / 6.0f;
  const float c = 1.0f / 6.0f;
  const float q0 = a * c;
  const float r = __builtin_fmaf(-q0, 6.0f, a);
  return __builtin_fmaf(r, c, q0);
}

// ---------------------------------------------------------------- E2M1
// Nearest-even magnitude code (0..7) of a >= 0; a >= 6 saturates to 7.
__device__ __forceinline__ uint32_t e2m1_rn_mag(float a) {
  if (a < 1.0f) return (uint32_t)__builtin_rintf(a + a);   // step 0.5: codes 0, 1, 2
  const uint32_t b = __float_as_uint(a);
  const uint32_t r = (b + 0x1FFFFFu + ((b >> 22) & 1u)) >> 22;   // keep 1 mantissa bit
  const uint32_t c = r - 252u;                                     // 1.0 -> code 2
  return c < 7u ? c : 7u;
}

// Stochastic E2M1 codes of 16 values with the hardware stochastic fp4 conversion.
//
// The rule (stochastic rounding of [NV-blog] recipe section bullet 5 with 16-bit draws):
// |a| rounds up to its upper grid neighbour iff (k + 1/2) / 2^16 < frac, frac being the
// position of |a| between its two neighbours; in units of 2^-22 of the grid step,
// F = frac * 2^22, that is F > 32 (2k + 1).
//
// v_cvt_scalef32_sr_pk_fp4_f32 converts a pair; for the value in position 0 it adds bits
// 10..31 of its 32-bit draw operand to the value's fraction of the fp4 step at 2^-22
// resolution and rounds up on the carry out of that field; it keeps the sign and
// saturates at 6 (found by recording the instruction on random inputs, then checked value
// by value against the rule at every decision point of every k: tests/test_gpu_conversions).
// So:
//  * the draw operand carries 2^22 - 1 - 32 (2k + 1) = 0x3FFFDF - 64k in bits 10..31: the
//    carry happens iff F + that >= 2^22, iff F >= 64k + 33, iff F > 64k + 32;
//  * F is an integer for |a| >= 1 (22 mantissa bits lie below the fp4 grid there), but
//    below 1 it may not be, so |a| is first rounded up to a multiple of 2^-23, which turns
//    F into ceil(F) without changing any decision (ceil(F) >= n + 1 iff F > n for an
//    integer n).  The caller passes t = a * 2^23 (exact: |a| < 2^104), the rounding up is
//    ceil(|t|) with the sign of t, and the conversion's scale operand 2^23 divides it
//    back exactly (a power of two);
//  * each element takes a conversion of its own (position 1 holds +0, code 0 for any
//    draw, because the two positions read overlapping draw bits): even elements fill the
//    bytes of one word, odd elements the bytes of another, shifted up a nibble.  The
//    conversion writes one byte of its destination and keeps the other three; the
//    compiler's builtin for it does not tie the destination to its "old" operand (it gives
//    each call a fresh register, losing the bytes written before), so the instruction is
//    issued through inline assembly with the destination as an in-out operand.
// w[j / 2] holds element j's draw: its low 16 bits for even j, its high 16 bits for odd j.
template <int BYTE>
__device__ __forceinline__ uint32_t cvt_sr_fp4_into(uint32_t acc, float2_t p, uint32_t r,
                                                    float scale) {
  if constexpr (BYTE == 0)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3" : "+v"(acc) : "v"(p), "v"(r), "s"(scale));
  else if constexpr (BYTE == 1)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,0]"
        : "+v"(acc) : "v"(p), "v"(r), "s"(scale));
  else if constexpr (BYTE == 2)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,0,1]"
        : "+v"(acc) : "v"(p), "v"(r), "s"(scale));
  else
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,1]"
        : "+v"(acc) : "v"(p), "v"(r), "s"(scale));
  return acc;
}

__device__ __forceinline__ uint2 e2m1_sr_pack16(const float t[16], const uint32_t w[8]) {
  uint32_t ev[2] = {0u, 0u}, od[2] = {0u, 0u};
  const float scale = 0x1p23f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float c = __builtin_copysignf(__builtin_ceilf(__builtin_fabsf(t[j])), t[j]);
    const uint32_t k16 = (j & 1) ? (w[j >> 1] & 0xFFFF0000u) : (w[j >> 1] << 16);   // k << 16
    const uint32_t r = 0xFFFF7C00u - k16;   // (0x3FFFDF - 64 k) << 10 | 0
    const float2_t p = {c, 0.0f};
    uint32_t &acc = (j & 1) ? od[j >> 3] : ev[j >> 3];
    switch ((j >> 1) & 3) {   // byte of the word (an immediate of the instruction)
      case 0: acc = cvt_sr_fp4_into<0>(acc, p, r, scale); break;
      case 1: acc = cvt_sr_fp4_into<1>(acc, p, r, scale); break;
      case 2: acc = cvt_sr_fp4_into<2>(acc, p, r, scale); break;
      default: acc = cvt_sr_fp4_into<3>(acc, p, r, scale); break;
    }
  }
  return make_uint2(ev[0] | (od[0] << 4), ev[1] | (od[1] << 4));
}

// Nearest-even E2M1 codes of 16 values y[j] * rr, packed two per byte (element 2i in
// the low nibble of byte i).  v_cvt_scalef32_pk_fp4_f32 with scale 1.0 rounds to
// nearest-even, saturates to +-6 and keeps the sign (including -0), which is exactly the
// encoder above; each instruction converts two values into one byte of the result.
__device__ __forceinline__ uint2 e2m1_rn_pack16(const float y[16], float rr) {
  uint32_t lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, y[0] * rr, y[1] * rr, 1.0f, 0);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, y[2] * rr, y[3] * rr, 1.0f, 1);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, y[4] * rr, y[5] * rr, 1.0f, 2);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, y[6] * rr, y[7] * rr, 1.0f, 3);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, y[8] * rr, y[9] * rr, 1.0f, 0);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, y[10] * rr, y[11] * rr, 1.0f, 1);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, y[12] * rr, y[13] * rr, 1.0f, 2);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, y[14] * rr, y[15] * rr, 1.0f, 3);
  return make_uint2(lo, hi);
}

// ---------------------------------------------------------------- decoding

// The two E2M1 codes of byte B of w (low nibble first) as fp32, exact: the hardware fp4
// conversion with scale 1.0.
template <int B>
__device__ __forceinline__ float2_t e2m1_decode_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
}

// Eight E2M1 codes (one dword, element 2i in the low nibble of byte i) times the block
// scale sbd, as eight fp16 values: the hardware fp4 -> fp16 conversion with scale 1.0, then
// a packed fp16 multiply.  Exact: every e2m1 * e4m3 product fits fp16 (at most 6
// significant bits, magnitudes 2^-10 .. 2688).
__device__ __forceinline__ half8_t dequant8_f16(uint32_t w, _Float16 sbd) {
  const half2_t s2 = {sbd, sbd};
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  half8_t r;
  r[0] = p0.x; r[1] = p0.y; r[2] = p1.x; r[3] = p1.y;
  r[4] = p2.x; r[5] = p2.y; r[6] = p3.x; r[7] = p3.y;
  return r;
}

// E4M3 bytes 2h and 2h+1 of w as two fp16 values (exact: the hardware fp8 -> fp16
// conversion with scale 1.0; every E4M3 value is an fp16 value).
__device__ __forceinline__ half2_t e4m3_pair_f16(uint32_t w, int h) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w >> (16 * h), 1.0f, false);
}

// bf16 bit pattern of v, nearest-even (the hardware conversion; NaN stays NaN).
__device__ __forceinline__ uint16_t bf16_bits_rn(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// ---------------------------------------------------------------- Philox4x32-10
// Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).
struct Philox4 { uint32_t x, y, z, w; };

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                  uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    // a ^ b ^ c in one instruction (truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32(hi1, c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32(hi0, c3, k1, 0x96);
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return Philox4{c0, c1, c2, c3};
}

// ---------------------------------------------------------------- buffer resources
// Raw buffer resource over `bytes` bytes at p: loads past the end return zero (clamped to
// 2^31 - 1 bytes; callers base it where the 32-bit offsets stay below that).  Every field is
// made wave-uniform so the descriptor lives in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *p, int64_t bytes) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF));
  return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0, n,
                                           0x00020000);
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// ---------------------------------------------------------------- lane exchange
// Partner lane l ^ D inside a row of 16 lanes: DPP quad permutations for D = 1, 2, a row
// rotation by 8 for D = 8 (the same as xor within 16 lanes) and ds_swizzle for D = 4.
__device__ __forceinline__ uint32_t lane_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
}
__device__ __forceinline__ uint32_t lane_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
}
__device__ __forceinline__ uint32_t lane_xor4(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x101F);              // and 0x1F, xor 4
}
__device__ __forceinline__ uint32_t lane_xor8(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false); // row_ror 8
}
template <int D>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  return D == 1 ? lane_xor1(v) : D == 2 ? lane_xor2(v) : D == 4 ? lane_xor4(v) : lane_xor8(v);
}

// Max over the 16 lanes of a DPP row (lanes 16q .. 16q+15).
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, lane_xor1(v));
  v = max(v, lane_xor2(v));
  v = max(v, lane_xor4(v));
  v = max(v, lane_xor8(v));
  return v;
}

// One butterfly stage of the 4-bit transpose, within each dword: a lane whose bit D is
// clear keeps the nibbles at positions p with (p & D) == 0 and takes its partner's,
// moved up by 4D bits; a lane with bit D set keeps the others and takes its partner's,
// moved down.  The rotation leaves wrapped bits only where the mask discards them.
template <int D>
__device__ __forceinline__ uint32_t nibble_stage(uint32_t w, bool hi_lane) {
  constexpr uint32_t s = 4 * D;
  constexpr uint32_t m0 = D == 4 ? 0x0000FFFFu : D == 2 ? 0x00FF00FFu : 0x0F0F0F0Fu;
  const uint32_t send = __builtin_amdgcn_alignbit(w, w, hi_lane ? 32 - s : s);  // rotate right
  const uint32_t recv = lane_xor<D>(send);
  const uint32_t keep = hi_lane ? ~m0 : m0;
  return (w & keep) | (recv & ~keep);
}

// 16 x 16 transpose of 4-bit codes across the 16 lanes of a DPP row.  On entry lane r
// holds row r (lo: columns 0..7, hi: columns 8..15, column c in nibble c % 8); on exit
// lane r holds column r (rows 0..7 in lo, rows 8..15 in hi).  Four butterfly stages
// swap bit D of the row index with bit D of the column index, D = 8, 4, 2, 1.
__device__ __forceinline__ void transpose_nibbles16(uint32_t &lo, uint32_t &hi, uint32_t r) {
  const bool b8 = r & 8;
  const uint32_t recv = lane_xor8(b8 ? lo : hi);
  lo = b8 ? recv : lo;
  hi = b8 ? hi : recv;
  lo = nibble_stage<4>(lo, r & 4);
  hi = nibble_stage<4>(hi, r & 4);
  lo = nibble_stage<2>(lo, r & 2);
  hi = nibble_stage<2>(hi, r & 2);
  lo = nibble_stage<1>(lo, r & 1);
  hi = nibble_stage<1>(hi, r & 1);
}

// Tensor scales from the tensor amax bit pattern (|y| as uint; >= 0x7F800000: non-finite).
struct TensorScale { float enc, dec; bool finite; };

__device__ __forceinline__ TensorScale tensor_scale(uint32_t amax_bits) {
  TensorScale t;
  t.finite = amax_bits < 0x7F800000u;
  const float amax = __uint_as_float(amax_bits);
  if (!t.finite) {
    t.enc = 1.0f;
    t.dec = __uint_as_float(0x7FC00000u);
  } else if (amax_bits == 0u) {
    t.enc = 1.0f;
    t.dec = 1.0f;
  } else {
    t.enc = fminf(kTensorRange / amax, kFltMax);
    t.dec = amax / kTensorRange;
  }
  return t;
}

// Per-element multiplier of a block whose decoded E4M3 scale is sbd.
__device__ __forceinline__ float block_mult(float s_enc, float sbd) {
  return sbd == 0.0f ? 0.0f : fminf(s_enc / sbd, kFltMax);
}

}  // namespace nvfp4
