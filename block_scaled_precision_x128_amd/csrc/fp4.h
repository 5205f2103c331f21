// Internal launcher interface of the FP4 (E2M1) microscaling kernels (host
// side, C++ linkage).  The public C ABI in include/fp8blk.h validates
// arguments and calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

enum { FP4_MX = 0, FP4_NV = 1 };

// Partial maxima of the NVFP4 tensor amax: at most kFp4Partials floats of workspace.
constexpr int kFp4Partials = 8192;

// x [rows, cols] fp32/bf16 (dt 0/1), cols % 128 == 0.  q: [rows, cols/2]
// packed codes; bs: MX [rows, cols/32] UE8M0 bytes, NV [rows, cols/16] E4M3
// microscale codes; ts: NV tensor scale (1 float); ws: NV partial maxima.
hipError_t launch_fp4_quantize(const void* x, int dt, int64_t rows, int64_t cols, int kind, uint8_t* q,
                               uint8_t* bs, float* ts, float* ws, hipStream_t st);
hipError_t launch_fp4_dequantize(const uint8_t* q, const uint8_t* bs, const float* ts, int64_t rows, int64_t cols,
                                 int kind, void* y, int odt, hipStream_t st);

}  // namespace fp8blk
