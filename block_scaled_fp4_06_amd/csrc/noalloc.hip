// noalloc.hip -- nvfp4_quantize_noalloc: nvfp4_quantize with a library-owned workspace.
//
// For callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc): the quantization workspace lives in a
// file-scope device array, `scratch`, of exactly nvfp4_quantize_workspace_bytes() bytes,
// which covers every shape the ABI accepts.  Each GPU the library runs on holds its own
// copy of the array until the process ends.
//
// The array starts zero-filled (static storage of the loaded code object), which is all the
// workspace protocol of the quantizers needs: every launch leaves its counters at zero and
// tags its other words with a fresh launch tag, so one call's contents are never mistaken
// for the next one's.  All calls on one GPU share the array: calls that overlap in time on
// one GPU (concurrent streams, other host threads) race and must not be made.
//
// In host code `scratch` names a host-side stand-in, not device memory.  Its device address
// is taken once per device, with that device current, through hipGetSymbolAddress, and that
// address is what the kernels receive.
#include <atomic>
#include <mutex>

#include "launch.hpp"
#include "nvfp4.h"

namespace {

__device__ __align__(256) static uint8_t scratch[nvfp4::kWorkspaceBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_init;

// Device address of `scratch` on device `dev` (taken once, with that device current).
hipError_t scratch_on(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) {
    *out = p;
    return hipSuccess;
  }
  std::lock_guard<std::mutex> lock(g_init);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (e2 != hipSuccess) return e2;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" nvfp4_status nvfp4_quantize_noalloc(const uint16_t *x, int64_t rows, int64_t cols,
                                               int64_t ld_x, const nvfp4_quant_params *p,
                                               uint8_t *codes, uint8_t *scales,
                                               float *global_dec, uint8_t *codes_t,
                                               uint8_t *scales_t, uint32_t *dev_status,
                                               nvfp4_stream_t stream) {
  nvfp4::QuantLaunch q;
  const nvfp4_status st = nvfp4::check_quantize(x, rows, cols, ld_x, p, codes, scales,
                                                global_dec, codes_t, scales_t, dev_status, &q);
  if (st != NVFP4_OK) return st;
  // every accepted shape fits the array; the bound is checked all the same
  if (nvfp4::kCoordBytes + 8 * nvfp4::quantize_chunks(rows, cols, p->blocking, p->rounding) >
      nvfp4::kPartialsOffset)
    return NVFP4_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = 0;
  if (hipStreamGetDevice(s, &dev) != hipSuccess) return NVFP4_ERR_HIP;
  void *ws = nullptr;
  if (scratch_on(dev, &ws) != hipSuccess) return NVFP4_ERR_HIP;
  q.ws = ws;
  return nvfp4::launch_quantize(q, s) == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}
