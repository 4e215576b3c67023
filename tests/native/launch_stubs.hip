// launch_stubs.hip -- stand-ins for the kernel launchers of libnvfp4 (test only).
//
// Linked with the library's argument-checking layer (api.hip) in a host-only build under
// UndefinedBehaviorSanitizer, so that every entry point can be driven on a machine without
// a GPU: a call that passes the checks reaches one of these functions, which records what
// it was asked to launch and returns an error instead of launching anything.
#include "launch.hpp"

extern "C" {
// What the last stub received (read by abi_ubsan_main.cpp).
int stub_calls = 0;
int64_t stub_rows = -1, stub_cols = -1, stub_ld = -1;
}

namespace nvfp4 {

static hipError_t record(int64_t rows, int64_t cols, int64_t ld) {
  ++stub_calls;
  stub_rows = rows;
  stub_cols = cols;
  stub_ld = ld;
  return hipErrorNotSupported;
}

hipError_t launch_quantize(const QuantLaunch &q, hipStream_t) { return record(q.rows, q.cols, q.ld); }
hipError_t launch_dequantize(const DequantLaunch &d, hipStream_t) { return record(d.rows, d.cols, d.ld_y); }
hipError_t launch_gemm(const GemmLaunch &g, hipStream_t) { return record(g.M, g.N, g.ldc); }
hipError_t launch_mx_quantize(const MxQuantLaunch &q, hipStream_t) { return record(q.rows, q.cols, q.ld); }
hipError_t launch_mx_dequantize(const MxDequantLaunch &d, hipStream_t) { return record(d.rows, d.cols, d.ld_y); }
hipError_t launch_mx_gemm(const MxGemmLaunch &g, hipStream_t) { return record(g.M, g.N, g.ldc); }
hipError_t launch_transpose_bf16(const TransposeLaunch &t, hipStream_t) { return record(t.rows, t.cols, t.ld_x); }

}  // namespace nvfp4
