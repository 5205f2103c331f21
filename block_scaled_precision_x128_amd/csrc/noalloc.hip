// fp8_quantize_noalloc: fp8_quantize for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The only scratch fp8_quantize needs is the per-tensor
// amax partials (FP8_GRAN_TENSOR, at most kTensorPartials floats); here it is a
// file-scope device array that every call on a GPU shares.
//
// The array's name is a host-side stand-in in host code, not a device
// address: its device address is fetched once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// handed to kernels.
#include <mutex>

#include "fp8blk.h"
#include "kernels.h"

namespace fp8blk {
namespace {

constexpr size_t kScratchBytes = sizeof(float) * (size_t)kTensorPartials;   // 32 KiB
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (fetched on the first call
// on that device).
fp8_status_t scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FP8_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FP8_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return FP8_OK;
}

}  // namespace
}  // namespace fp8blk

extern "C" fp8_status_t fp8_quantize_noalloc(const void* x, fp8_dtype_t x_dt, int64_t rows, int64_t cols,
                                             fp8_format_t fmt, fp8_granularity_t g, uint8_t* q, void* scales,
                                             hipStream_t stream) {
  const size_t need = fp8_quantize_workspace_bytes(rows, cols, g);
  if (need > fp8blk::kScratchBytes) return FP8_ERR_WORKSPACE;   // beyond the static scratch
  // Every argument check of fp8_quantize runs before any HIP call; with no
  // workspace a valid call that needs one stops at FP8_ERR_WORKSPACE, having
  // enqueued nothing, and one that needs none is done.
  const fp8_status_t st = fp8_quantize(x, x_dt, rows, cols, fmt, g, q, scales, nullptr, 0, stream);
  if (st != FP8_ERR_WORKSPACE || need == 0) return st;
  void* ws = nullptr;
  const fp8_status_t sa = fp8blk::scratch_address(&ws);
  if (sa != FP8_OK) return sa;
  return fp8_quantize(x, x_dt, rows, cols, fmt, g, q, scales, ws, fp8blk::kScratchBytes, stream);
}
