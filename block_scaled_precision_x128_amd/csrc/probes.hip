// Measurement probes (include/fp8blk_probe.h): the matrix-core rate of
// back-to-back independent MFMAs, a streaming read and a device copy.  They
// give the ceilings the library's kernels are measured against beside the
// published peaks ("The FP8 Family", "What Hopper actually gives you": compute
// roof and ridge point; "FP8 Serving", "What FP8 actually buys": decode speed
// follows the bytes read).
#include "fp8blk.h"
#include "fp8blk_probe.h"
#include "gemm_common.h"

namespace fp8blk {

constexpr int kReadBlocks = 1024;    // workgroups of the read probe
constexpr int kCopyBlocks = 2048;    // workgroups of the copy probe
constexpr int kChains = 8;           // independent accumulators per wave

// Each wave issues `iters` rounds of kChains independent MFMAs on operands
// built from the thread index (values are irrelevant to the rate).
template <int KIND>
__global__ __launch_bounds__(512) void k_probe_mfma(float* sink, int iters) {
  const int t = threadIdx.x;
  v4f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (KIND == FP8BLK_PROBE_MFMA_BF16) {
    v8bf a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(float)((t + i) & 7);
      b[i] = (__bf16)(float)((3 * t + i) & 7);
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = mfma_bf16(a, b, acc[c]);
  } else {
    v8i a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x38383838 ^ ((t + i) & 0x07070707);   // E4M3 codes near 1.0
      b[i] = 0x30303030 ^ ((3 * t + i) & 0x07070707);
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = mfma_fp8<FMT_E4M3, FMT_E4M3>(a, b, acc[c], (int)kUnitScale, (int)kUnitScale);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  sink[(int64_t)blockIdx.x * blockDim.x + t] = s;
}

// Each workgroup streams one contiguous chunk, eight 16-byte loads in flight
// per thread (a grid-stride loop over the whole buffer measured 5.3 TB/s
// against 6.0 for contiguous chunks).
__global__ __launch_bounds__(256) void k_probe_read(const u32x4* src, int64_t n16, uint32_t* sink) {
  constexpr int U = 8;
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per, b1 = b0 + per < n16 ? b0 + per : n16;
  int64_t i = b0 + threadIdx.x;
  uint32_t x = 0;
  for (; i + (U - 1) * 256 < b1; i += U * 256) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * 256];
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < b1; i += 256) {
    const u32x4 v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = x;
}

// The same chunking, eight loads in flight, non-temporal loads and stores
// (5.57 TB/s of read + write against 5.3 with ordinary ones).
__global__ __launch_bounds__(256) void k_probe_copy(const u32x4* src, u32x4* dst, int64_t n16) {
  constexpr int U = 8;
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per, b1 = b0 + per < n16 ? b0 + per : n16;
  int64_t i = b0 + threadIdx.x;
  for (; i + (U - 1) * 256 < b1; i += U * 256) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(&src[i + u * 256]);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], &dst[i + u * 256]);
  }
  for (; i < b1; i += 256) dst[i] = src[i];
}

}  // namespace fp8blk

using namespace fp8blk;

extern "C" {

size_t fp8blk_probe_mfma_sink_floats(int waves_per_simd) {
  if (waves_per_simd < 1 || waves_per_simd > 2) return 0;
  return (size_t)num_cus() * 256u * (size_t)waves_per_simd;
}

int fp8blk_probe_mfma(int kind, int waves_per_simd, int iters, float* sink, double* flops, hipStream_t stream) {
  if (kind != FP8BLK_PROBE_MFMA_BF16 && kind != FP8BLK_PROBE_MFMA_FP8) return FP8_ERR_ENUM;
  if (waves_per_simd < 1 || waves_per_simd > 2 || iters < 1) return FP8_ERR_SHAPE;
  if (!sink || !flops) return FP8_ERR_NULL;
  const int cus = num_cus(), threads = 256 * waves_per_simd;
  const double per_inst = kind == FP8BLK_PROBE_MFMA_BF16 ? 2.0 * 16 * 16 * 32 : 2.0 * 16 * 16 * 128;
  *flops = per_inst * kChains * (double)iters * (threads / 64) * cus;
  if (kind == FP8BLK_PROBE_MFMA_BF16)
    hipLaunchKernelGGL(k_probe_mfma<FP8BLK_PROBE_MFMA_BF16>, dim3(cus), dim3(threads), 0, stream, sink, iters);
  else
    hipLaunchKernelGGL(k_probe_mfma<FP8BLK_PROBE_MFMA_FP8>, dim3(cus), dim3(threads), 0, stream, sink, iters);
  return hipGetLastError() == hipSuccess ? FP8_OK : FP8_ERR_HIP;
}

size_t fp8blk_probe_read_sink_floats(void) { return (size_t)kReadBlocks * 256u; }

int fp8blk_probe_read(const void* src, int64_t bytes, float* sink, hipStream_t stream) {
  if (!src || !sink) return FP8_ERR_NULL;
  if (bytes < 0 || bytes % 16 != 0) return FP8_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return FP8_ERR_ALIGN;
  hipLaunchKernelGGL(k_probe_read, dim3(kReadBlocks), dim3(256), 0, stream, static_cast<const u32x4*>(src),
                     bytes / 16, reinterpret_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? FP8_OK : FP8_ERR_HIP;
}

int fp8blk_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  if (!src || !dst) return FP8_ERR_NULL;
  if (bytes < 0 || bytes % 16 != 0) return FP8_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0) return FP8_ERR_ALIGN;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  if (s0 < d0 + (uintptr_t)bytes && d0 < s0 + (uintptr_t)bytes && bytes > 0) return FP8_ERR_SHAPE;
  hipLaunchKernelGGL(k_probe_copy, dim3(kCopyBlocks), dim3(256), 0, stream, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? FP8_OK : FP8_ERR_HIP;
}

}  // extern "C"
