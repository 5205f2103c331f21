// Internal launcher interface of libfp8blk (host side, C++ linkage).  The
// public C ABI in include/fp8blk.h validates arguments and calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

// Number of per-workgroup partial maxima of the per-tensor amax pass; the
// per-tensor quantize needs kTensorPartials floats of workspace.
constexpr int kTensorPartials = 8192;

enum { MODE_EPILOGUE = 0, MODE_PROMOTE = 1, MODE_MX = 2 };
// FP4 (E2M1, two codes per byte) operands: MXFP4 (UE8M0 per 32 K) and NVFP4
// (E4M3 microscale per 16 K, fp32 tensor scales ta, tb).
enum { MODE_MX4 = 3, MODE_NV4 = 4 };
// Kernel-internal form of MODE_MX4 for K % 512 == 0: a row's scale bytes of
// 256-K steps 2p and 2p+1 form one 16-byte aligned block, staged with one
// 16-byte load.
enum { MODE_MX4_PAIRS = 5 };
// Matrix-core path: exact products with fp32 sums (bf16 instructions on the
// expanded codes), or the FP8 instructions' own accumulation.
enum { PATH_EXACT = 0, PATH_FAST = 1 };
// GEMM output kinds beyond the public DT_F32 / DT_BF16: the result quantized
// in the epilogue to FP8 codes with one fp32 scale per 1x128 tile of a row.
enum { ODT_Q_E4M3 = 2, ODT_Q_E5M2 = 3 };

struct GemmArgs {
  const uint8_t* a;   // [M, K] codes
  const uint8_t* b;   // [N, K] codes
  const void* sa;     // scales of a (layout per granularity)
  const void* sb;     // scales of b
  void* out;          // [M, N] values, or codes for the quantized outputs
  float* out_scales;  // quantized outputs: [M, N/128] fp32 tile scales
  const float* ta;    // MODE_NV4: tensor scale of a (1 float)
  const float* tb;    // MODE_NV4: tensor scale of b
  int64_t M, N, K;
  int64_t ldo;        // elements between consecutive rows of out (>= N)
  int a_per_row;      // epilogue mode: 1 = one scale per row of a, 0 = one per tensor
  int b_per_row;      // epilogue mode: same for b
};

hipError_t launch_quantize(const void* x, int dt, int64_t rows, int64_t cols, int fmt, int g, uint8_t* q,
                           void* scales, void* ws, hipStream_t st);
// Delayed scaling of a whole tensor of `total` elements (total % 8 == 0):
// scale[0] from hist[0..len), codes under it, then hist[pos] = amax.
hipError_t launch_quantize_delayed(const void* x, int dt, int64_t total, int fmt, float* hist, int64_t len,
                                   int64_t pos, int margin, uint8_t* q, float* scale, void* ws, hipStream_t st);
hipError_t launch_cast(const void* x, int dt, int64_t n, int fmt, uint8_t* q, hipStream_t st);
hipError_t launch_dequantize(const uint8_t* q, const void* scales, int64_t rows, int64_t cols, int fmt, int g,
                             void* y, int odt, hipStream_t st);
hipError_t launch_gemm_tiled(const GemmArgs& p, int afmt, int bfmt, int mode, int odt, int path, hipStream_t st);
hipError_t launch_gemm_skinny(const GemmArgs& p, int afmt, int bfmt, int mode, int odt, int path, hipStream_t st);
// FP4 operands (mode MODE_MX4 or MODE_NV4, odt DT_F32 / DT_BF16, K % 256 == 0).
hipError_t launch_gemm_fp4(const GemmArgs& p, int mode, int odt, hipStream_t st);
// FP4 operands with M <= 64 (decode shapes): the skinny kernel (mode
// MODE_MX4 or MODE_NV4).
hipError_t launch_gemm_skinny_fp4(const GemmArgs& p, int mode, int odt, hipStream_t st);
hipError_t launch_fill_zero(void* out, int64_t bytes, hipStream_t st);     // bytes % 4 == 0, 4-byte aligned
hipError_t launch_fill_f32(float* out, int64_t n, float v, hipStream_t st);

}  // namespace fp8blk
