// FP8 dequantization for gfx950: y = RN32(decode(q) * s), MX: decode(q) * 2^e,
// optionally rounded to bf16 (nearest even).  ("The FP8 Family", dequant
// formula; "Illustrated GPU kernels, Part 8", the dequantization multiply of
// the qdq listing.)  A workgroup converts 4096 consecutive elements.  Each
// thread takes P pieces of 16/P elements (8 for bf16 output, 4 for fp32), at
// offsets (16/P)(t + 256 p), so that every 16-byte output store is contiguous
// across the wave: stores at a 32- or 64-byte lane stride (16 contiguous
// elements per thread) measured 15-25% slower on this write-heavy stream.
// A piece never straddles a scale group (groups are multiples of 32 elements,
// rows multiples of 128).
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
  constexpr int P = ODT == DT_F32 ? 4 : 2;
  constexpr int E = 16 / P;
  const int64_t base = (int64_t)blockIdx.x * 4096;
  int64_t row0 = 0, col0 = 0;
  if constexpr (G == G_ROW || G == G_BLOCK) {
    row0 = base / cols;
    col0 = base - row0 * cols;
  }
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int off = E * ((int)threadIdx.x + 256 * p);
    const int64_t e0 = base + off;
    if (e0 >= total) break;   // total is a multiple of 128: pieces lie wholly inside or outside
    float s = 1.0f;
    int e = 0;
    bool nan_scale = false;
    if constexpr (G == G_TENSOR) {
      s = reinterpret_cast<const float*>(scales)[0];
    } else if constexpr (G == G_TILE) {
      s = reinterpret_cast<const float*>(scales)[e0 / 128];
    } else if constexpr (G == G_MX) {
      const uint32_t b = reinterpret_cast<const uint8_t*>(scales)[e0 / 32];
      e = (int)b - 127;
      nan_scale = (b == 255u);
    } else {
      int64_t row = row0, col = col0 + off;
      if (col >= cols) {   // the piece lies in a later row than the workgroup's first element
        const int64_t k = col / cols;
        row += k;
        col -= k * cols;
      }
      if constexpr (G == G_ROW) s = reinterpret_cast<const float*>(scales)[row];
      else s = reinterpret_cast<const float*>(scales)[(row / 128) * (cols / 128) + col / 128];
    }
    uint32_t w[E / 4];
    if constexpr (E == 8) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(q + e0);
      w[0] = v.x;
      w[1] = v.y;
    } else {
      w[0] = *reinterpret_cast<const uint32_t*>(q + e0);
    }
    float v[E];
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const v2f lo = decode2<FMT>(w[i], false), hi = decode2<FMT>(w[i], true);
      v[4 * i] = lo.x; v[4 * i + 1] = lo.y; v[4 * i + 2] = hi.x; v[4 * i + 3] = hi.y;
    }
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if constexpr (G == G_MX) v[i] = nan_scale ? __builtin_nanf("") : __builtin_amdgcn_ldexpf(v[i], e);
      else v[i] = v[i] * s;
    }
    if constexpr (ODT == DT_F32) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + e0) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(y) + e0) =
          u32x4{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
    }
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
  const dim3 grid((unsigned)((total + 4095) / 4096));
  if (fmt == FMT_E4M3) dequant_f<FMT_E4M3>(q, scales, cols, total, y, g, odt, grid, st);
  else dequant_f<FMT_E5M2>(q, scales, cols, total, y, g, odt, grid, st);
  return hipGetLastError();
}

}  // namespace fp8blk
