// transpose.hip -- bf16 transpose for gfx950.
//
// The weight-gradient product of a linear layer contracts over the token dimension M:
// dW = X^T dY (NVIDIA developer blog zh-cn "NVFP4 trains with precision of 16-bit ...",
// section "用于预训练的 NVFP4 量化配方": the Hadamard transform and the quantization are
// applied to the GEMM inputs in the backward pass as well).  Quantizing X^T and dY^T along
// M needs them with M contiguous; this kernel writes them.  HBM-bound: 2 bytes read and 2
// written per element.
//
// A 64 x 64 tile per 256-thread workgroup: each thread loads two 16-byte pieces (8
// elements of a row), the tile goes through LDS with rows padded by 8 elements (so the
// column gathers of one wave spread over the banks), and each thread writes two 16-byte
// pieces of the transposed rows.  Rows and columns are multiples of 8; tiles past the
// edge are masked per 8-element piece.  Consecutive workgroups take consecutive tiles down
// a tile column, so the workgroups in flight complete long runs of each output row (8 %
// faster than walking along the input rows on an 8192 x 20480 transpose).
#include "launch.hpp"

namespace nvfp4 {
namespace {

constexpr int kTT = 64;          // tile edge
constexpr int kTPad = kTT + 8;   // LDS row stride in elements

__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t *__restrict__ x,
                                                             int64_t rows, int64_t cols, int64_t ld_x,
                                                             uint16_t *__restrict__ y, int64_t ld_y,
                                                             int tiles_r) {
  __shared__ __attribute__((aligned(16))) uint16_t t[kTT * kTPad];
  const int64_t r0 = (int64_t)(blockIdx.x % tiles_r) * kTT;
  const int64_t c0 = (int64_t)(blockIdx.x / tiles_r) * kTT;
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int piece = tid + 256 * k;            // 512 pieces of 8 elements
    const int lr = piece >> 3, lc = (piece & 7) * 8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r0 + lr < rows && c0 + lc < cols)
      v = *reinterpret_cast<const uint4 *>(x + (r0 + lr) * ld_x + c0 + lc);
    *reinterpret_cast<uint4 *>(t + lr * kTPad + lc) = v;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int piece = tid + 256 * k;
    const int oc = piece >> 3, orow = (piece & 7) * 8;   // output row c0 + oc, columns r0 + orow ..
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)t[(orow + 2 * j) * kTPad + oc] | ((uint32_t)t[(orow + 2 * j + 1) * kTPad + oc] << 16);
    if (c0 + oc < cols && r0 + orow < rows)
      *reinterpret_cast<uint4 *>(y + (c0 + oc) * ld_y + r0 + orow) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

hipError_t launch_transpose_bf16(const TransposeLaunch &t, hipStream_t stream) {
  if (t.rows == 0 || t.cols == 0) return hipSuccess;
  const int64_t tr = (t.rows + kTT - 1) / kTT, tc = (t.cols + kTT - 1) / kTT;
  transpose_bf16_kernel<<<(uint32_t)(tr * tc), 256, 0, stream>>>(t.x, t.rows, t.cols, t.ld_x, t.y,
                                                                 t.ld_y, (int)tr);
  return hipGetLastError();
}

}  // namespace nvfp4
