// FP8 dequantization for gfx950: y = RN32(decode(q) * s), MX: decode(q) * 2^e,
// optionally rounded to bf16 (nearest even).  ("The FP8 Family", dequant
// formula; "Illustrated GPU kernels, Part 8", the dequantization multiply of
// the qdq listing.)  Each thread turns 16 codes (one 16-byte load) into 16
// outputs; 16 consecutive elements never straddle a scale group.
#include "device_common.h"
#include "kernels.h"

namespace fp8blk {

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

template <int FMT, int G, int ODT>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ q, const void* __restrict__ scales,
                                                  int64_t cols, int64_t total, void* __restrict__ y) {
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 16;
  if (e0 >= total) return;
  float s = 1.0f;
  int e = 0;
  bool nan_scale = false;
  if constexpr (G == G_TENSOR) {
    s = reinterpret_cast<const float*>(scales)[0];
  } else if constexpr (G == G_ROW) {
    s = reinterpret_cast<const float*>(scales)[e0 / cols];
  } else if constexpr (G == G_TILE) {
    s = reinterpret_cast<const float*>(scales)[e0 / 128];
  } else if constexpr (G == G_BLOCK) {
    const int64_t row = e0 / cols, col = e0 - row * cols;
    s = reinterpret_cast<const float*>(scales)[(row / 128) * (cols / 128) + col / 128];
  } else {
    const uint32_t b = reinterpret_cast<const uint8_t*>(scales)[e0 / 32];
    e = (int)b - 127;
    nan_scale = (b == 255u);
  }
  const u32x4 w = *reinterpret_cast<const u32x4*>(q + e0);
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v2f lo = decode2<FMT>(ws[i], false), hi = decode2<FMT>(ws[i], true);
    v[4 * i] = lo.x; v[4 * i + 1] = lo.y; v[4 * i + 2] = hi.x; v[4 * i + 3] = hi.y;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if constexpr (G == G_MX) v[i] = nan_scale ? __builtin_nanf("") : __builtin_amdgcn_ldexpf(v[i], e);
    else v[i] = v[i] * s;
  }
  if constexpr (ODT == DT_F32) {
    float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + e0);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  } else {
    u32x4* dst = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(y) + e0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dst[i] = u32x4{pack_bf16(v[8 * i], v[8 * i + 1]), pack_bf16(v[8 * i + 2], v[8 * i + 3]),
                     pack_bf16(v[8 * i + 4], v[8 * i + 5]), pack_bf16(v[8 * i + 6], v[8 * i + 7])};
  }
}

template <int FMT, int G>
static void dequant_g(const uint8_t* q, const void* sc, int64_t cols, int64_t total, void* y, int odt, dim3 grid,
                      hipStream_t st) {
  if (odt == DT_F32)
    hipLaunchKernelGGL((k_dequant<FMT, G, DT_F32>), grid, dim3(256), 0, st, q, sc, cols, total, y);
  else
    hipLaunchKernelGGL((k_dequant<FMT, G, DT_BF16>), grid, dim3(256), 0, st, q, sc, cols, total, y);
}

template <int FMT>
static void dequant_f(const uint8_t* q, const void* sc, int64_t cols, int64_t total, void* y, int g, int odt,
                      dim3 grid, hipStream_t st) {
  switch (g) {
    case G_TENSOR: dequant_g<FMT, G_TENSOR>(q, sc, cols, total, y, odt, grid, st); break;
    case G_ROW: dequant_g<FMT, G_ROW>(q, sc, cols, total, y, odt, grid, st); break;
    case G_TILE: dequant_g<FMT, G_TILE>(q, sc, cols, total, y, odt, grid, st); break;
    case G_BLOCK: dequant_g<FMT, G_BLOCK>(q, sc, cols, total, y, odt, grid, st); break;
    default: dequant_g<FMT, G_MX>(q, sc, cols, total, y, odt, grid, st); break;
  }
}

hipError_t launch_dequantize(const uint8_t* q, const void* scales, int64_t rows, int64_t cols, int fmt, int g,
                             void* y, int odt, hipStream_t st) {
  const int64_t total = rows * cols;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total / 16 + 255) / 256));
  if (fmt == FMT_E4M3) dequant_f<FMT_E4M3>(q, scales, cols, total, y, g, odt, grid, st);
  else dequant_f<FMT_E5M2>(q, scales, cols, total, y, g, odt, grid, st);
  return hipGetLastError();
}

}  // namespace fp8blk
