// Internal launcher interface of the FP8 KV-cache kernels (host side, C++
// linkage).  The public C ABI in include/fp8blk.h validates arguments and
// calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

// Rows of L = heads * head_dim elements (head_dim % 16 == 0); sk: 0 per
// tensor, 1 per head, 2 per channel; dt / odt: 0 fp32, 1 bf16.  Slots
// outside [0, num_slots) are skipped on append and read as zeros.
hipError_t launch_kv_append(const void* x, int dt, int64_t ld_x, const int64_t* slots, int64_t tokens, int fmt,
                            int sk, const float* scales, int head_dim, int64_t L, uint8_t* cache, int64_t num_slots,
                            hipStream_t st);
hipError_t launch_kv_gather(const uint8_t* cache, int64_t num_slots, const int64_t* slots, int64_t n, int fmt, int sk,
                            const float* scales, int head_dim, int64_t L, void* out, int odt, hipStream_t st);

}  // namespace fp8blk
