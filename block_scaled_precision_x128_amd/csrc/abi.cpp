// C ABI of libfp8blk: argument validation on the host, then kernel selection
// and launch on the caller's stream.  Declarations and the meaning of every
// argument are in include/fp8blk.h.
#include "../../include/fp8blk.h"

#include <limits.h>

#include "fp4.h"
#include "kernels.h"
#include "kv_cache.h"

using namespace fp8blk;

namespace {

// Largest GEMM K: the kernels address up to 256 operand rows (256 * K bytes)
// plus an out-of-range sentinel through 32-bit buffer offsets.
constexpr int64_t kMaxGemmK = int64_t(1) << 22;

bool valid_fmt(fp8_format_t f) { return f == FP8_E4M3 || f == FP8_E5M2; }
bool valid_dt(fp8_dtype_t d) { return d == FP8_DT_F32 || d == FP8_DT_BF16; }
bool valid_gran(fp8_granularity_t g) { return g >= FP8_GRAN_TENSOR && g <= FP8_GRAN_MX32; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Product of two non-negative sizes, or -1 if it overflows.
int64_t mul_checked(int64_t a, int64_t b) {
  if (a == 0 || b == 0) return 0;
  if (a > INT64_MAX / b) return -1;
  return a * b;
}

fp8_status_t check_operand(int64_t rows, int64_t cols, fp8_granularity_t g) {
  if (rows < 0 || cols < 0) return FP8_ERR_SHAPE;
  if (cols % 128 != 0) return FP8_ERR_SHAPE;
  if (g == FP8_GRAN_BLOCK_128x128 && rows % 128 != 0) return FP8_ERR_SHAPE;
  const int64_t total = mul_checked(rows, cols);
  if (total < 0) return FP8_ERR_SHAPE;
  // every launch below keeps its grid under 2^31 workgroups
  if (total / 32 / 256 >= INT_MAX || rows >= INT_MAX) return FP8_ERR_SHAPE;
  return FP8_OK;
}

fp8_status_t hip_status(hipError_t e) { return e == hipSuccess ? FP8_OK : FP8_ERR_HIP; }

// Largest KV-cache row (heads * head_dim elements).
constexpr int64_t kMaxKvRow = int64_t(1) << 24;

bool valid_fp4(fp4_scaling_t k) { return k == FP4_SCALE_MX || k == FP4_SCALE_NV; }

bool valid_kv_scale(fp8_kv_scale_t k) { return k >= FP8_KV_SCALE_TENSOR && k <= FP8_KV_SCALE_CHANNEL; }

// Row length L = heads * head_dim of a KV cache, or -1 for an invalid shape.
int64_t kv_row(int64_t heads, int64_t head_dim) {
  if (heads < 0 || head_dim < 0 || head_dim % 16 != 0) return -1;
  if (heads > 0 && head_dim > kMaxKvRow / heads) return -1;
  return heads * head_dim;
}

}  // namespace

extern "C" {

const char* fp8_status_string(fp8_status_t st) {
  switch (st) {
    case FP8_OK: return "ok";
    case FP8_ERR_NULL: return "a required pointer is NULL";
    case FP8_ERR_ENUM: return "invalid format, granularity, dtype or algorithm value";
    case FP8_ERR_SHAPE: return "invalid shape (negative, K % 128, rows % 128 for 128x128 blocks, M/N % 16, GEMM K > 2^22, KV head_dim % 16 or row stride, or too large)";
    case FP8_ERR_UNSUPPORTED: return "unsupported combination";
    case FP8_ERR_WORKSPACE: return "workspace missing or too small";
    case FP8_ERR_HIP: return "HIP launch failed";
    case FP8_ERR_ALIGN: return "misaligned pointer (tensors need 16 bytes, fp32 scales 4 bytes)";
  }
  return "unknown status";
}

int fp8_abi_version(void) { return FP8BLK_ABI_VERSION; }

size_t fp8_quantize_workspace_bytes(int64_t rows, int64_t cols, fp8_granularity_t g) {
  if (!valid_gran(g) || check_operand(rows, cols, g) != FP8_OK) return 0;
  return g == FP8_GRAN_TENSOR ? sizeof(float) * (size_t)kTensorPartials : 0;
}

fp8_status_t fp8_quantize(const void* x, fp8_dtype_t x_dt, int64_t rows, int64_t cols, fp8_format_t fmt,
                          fp8_granularity_t g, uint8_t* q, void* scales, void* workspace, size_t ws_bytes,
                          hipStream_t stream) {
  if (!valid_dt(x_dt) || !valid_fmt(fmt) || !valid_gran(g)) return FP8_ERR_ENUM;
  const fp8_status_t sh = check_operand(rows, cols, g);
  if (sh != FP8_OK) return sh;
  const int64_t total = rows * cols;
  if (total > 0 && (!x || !q)) return FP8_ERR_NULL;
  if ((total > 0 || g == FP8_GRAN_TENSOR) && !scales) return FP8_ERR_NULL;
  if (total > 0 && (!aligned(x, 16) || !aligned(q, 16))) return FP8_ERR_ALIGN;
  if (g != FP8_GRAN_MX32 && scales && !aligned(scales, 4)) return FP8_ERR_ALIGN;
  if (g == FP8_GRAN_TENSOR && total > 0) {
    if (!workspace || ws_bytes < sizeof(float) * (size_t)kTensorPartials) return FP8_ERR_WORKSPACE;
    if (!aligned(workspace, 4)) return FP8_ERR_ALIGN;
  }
  return hip_status(launch_quantize(x, (int)x_dt, rows, cols, (int)fmt, (int)g, q, scales, workspace, stream));
}

fp8_status_t fp8_quantize_delayed(const void* x, fp8_dtype_t x_dt, int64_t rows, int64_t cols, fp8_format_t fmt,
                                  float* history, int64_t hist_len, int64_t hist_pos, int margin, uint8_t* q,
                                  float* scale, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dt(x_dt) || !valid_fmt(fmt)) return FP8_ERR_ENUM;
  const fp8_status_t sh = check_operand(rows, cols, FP8_GRAN_TENSOR);
  if (sh != FP8_OK) return sh;
  if (hist_len < 1 || hist_len > (int64_t(1) << 30) || hist_pos < 0 || hist_pos >= hist_len) return FP8_ERR_SHAPE;
  if (margin < 0 || margin > 31) return FP8_ERR_SHAPE;
  const int64_t total = rows * cols;
  if (!history || !scale) return FP8_ERR_NULL;
  if (!aligned(history, 4) || !aligned(scale, 4)) return FP8_ERR_ALIGN;
  if (total > 0) {
    if (!x || !q) return FP8_ERR_NULL;
    if (!aligned(x, 16) || !aligned(q, 16)) return FP8_ERR_ALIGN;
    if (!workspace || ws_bytes < sizeof(float) * (size_t)kTensorPartials) return FP8_ERR_WORKSPACE;
    if (!aligned(workspace, 4)) return FP8_ERR_ALIGN;
  }
  return hip_status(launch_quantize_delayed(x, (int)x_dt, total, (int)fmt, history, hist_len, hist_pos, margin, q,
                                            scale, workspace, stream));
}

fp8_status_t fp8_dequantize(const uint8_t* q, const void* scales, int64_t rows, int64_t cols, fp8_format_t fmt,
                            fp8_granularity_t g, void* y, fp8_dtype_t y_dt, hipStream_t stream) {
  if (!valid_dt(y_dt) || !valid_fmt(fmt) || !valid_gran(g)) return FP8_ERR_ENUM;
  const fp8_status_t sh = check_operand(rows, cols, g);
  if (sh != FP8_OK) return sh;
  const int64_t total = rows * cols;
  if (total == 0) return FP8_OK;
  if (!q || !scales || !y) return FP8_ERR_NULL;
  if (!aligned(q, 16) || !aligned(y, 16)) return FP8_ERR_ALIGN;
  if (g != FP8_GRAN_MX32 && !aligned(scales, 4)) return FP8_ERR_ALIGN;
  return hip_status(launch_dequantize(q, scales, rows, cols, (int)fmt, (int)g, y, (int)y_dt, stream));
}

fp8_status_t fp8_cast(const void* x, fp8_dtype_t x_dt, int64_t n, fp8_format_t fmt, uint8_t* q,
                      hipStream_t stream) {
  if (!valid_dt(x_dt) || !valid_fmt(fmt)) return FP8_ERR_ENUM;
  if (n < 0 || n % 8 != 0 || n / 8 / 256 >= INT_MAX) return FP8_ERR_SHAPE;
  if (n == 0) return FP8_OK;
  if (!x || !q) return FP8_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 8)) return FP8_ERR_ALIGN;
  return hip_status(launch_cast(x, (int)x_dt, n, (int)fmt, q, stream));
}

namespace {

// Validation and mode selection shared by the GEMM entry points; fills p
// (without the output) and the scale mode.  Returns FP8_OK or an error.
static fp8_status_t gemm_common(const uint8_t* a, fp8_format_t a_fmt, fp8_granularity_t a_g, const void* a_scales,
                         const uint8_t* b, fp8_format_t b_fmt, fp8_granularity_t b_g, const void* b_scales,
                         int64_t M, int64_t N, int64_t K, fp8_accum_t accum, GemmArgs& p, int& mode) {
  if (!valid_fmt(a_fmt) || !valid_fmt(b_fmt) || !valid_gran(a_g) || !valid_gran(b_g)) return FP8_ERR_ENUM;
  if (accum != FP8_ACCUM_FP32 && accum != FP8_ACCUM_NATIVE) return FP8_ERR_ENUM;
  if (M < 0 || N < 0 || K < 0 || M % 16 || N % 16 || K % 128) return FP8_ERR_SHAPE;
  if (K > kMaxGemmK) return FP8_ERR_SHAPE;
  if (mul_checked(M, K) < 0 || mul_checked(N, K) < 0 || mul_checked(M, N) < 0) return FP8_ERR_SHAPE;
  if ((M / 128 + 1) * (N / 128 + 1) >= INT_MAX || N / 16 >= INT_MAX) return FP8_ERR_SHAPE;
  const bool a_tr = (a_g == FP8_GRAN_TENSOR || a_g == FP8_GRAN_ROW);
  const bool b_tr = (b_g == FP8_GRAN_TENSOR || b_g == FP8_GRAN_ROW);
  if (a_tr && b_tr) mode = MODE_EPILOGUE;
  else if (a_g == FP8_GRAN_TILE_1x128 && b_g == FP8_GRAN_BLOCK_128x128) mode = MODE_PROMOTE;
  else if (a_g == FP8_GRAN_MX32 && b_g == FP8_GRAN_MX32) mode = MODE_MX;
  else return FP8_ERR_UNSUPPORTED;
  if (b_g == FP8_GRAN_BLOCK_128x128 && N % 128) return FP8_ERR_SHAPE;
  p = GemmArgs{};
  p.a = a;
  p.b = b;
  p.sa = a_scales;
  p.sb = b_scales;
  p.M = M;
  p.N = N;
  p.K = K;
  p.ldo = N;
  p.a_per_row = (a_g == FP8_GRAN_ROW);
  p.b_per_row = (b_g == FP8_GRAN_ROW);
  return FP8_OK;
}

static fp8_status_t check_operands(const GemmArgs& p) {
  if (!p.a || !p.b || !p.sa || !p.sb) return FP8_ERR_NULL;
  if (!aligned(p.a, 16) || !aligned(p.b, 16)) return FP8_ERR_ALIGN;
  // fp32 scales are read as floats; UE8M0 scales as 4-byte words (4 blocks of 32)
  if (!aligned(p.sa, 4) || !aligned(p.sb, 4)) return FP8_ERR_ALIGN;
  return FP8_OK;
}

}  // namespace

fp8_status_t fp8_gemm_blockscaled_ex(const uint8_t* a, fp8_format_t a_fmt, fp8_granularity_t a_g,
                                     const void* a_scales, const uint8_t* b, fp8_format_t b_fmt,
                                     fp8_granularity_t b_g, const void* b_scales, int64_t M, int64_t N, int64_t K,
                                     void* out, fp8_dtype_t out_dt, fp8_gemm_algo_t algo, fp8_accum_t accum,
                                     hipStream_t stream) {
  if (!valid_dt(out_dt)) return FP8_ERR_ENUM;
  if (algo != FP8_GEMM_AUTO && algo != FP8_GEMM_TILED && algo != FP8_GEMM_SKINNY) return FP8_ERR_ENUM;
  GemmArgs p;
  int mode = 0;
  const fp8_status_t st = gemm_common(a, a_fmt, a_g, a_scales, b, b_fmt, b_g, b_scales, M, N, K, accum, p, mode);
  if (st != FP8_OK) return st;
  if (algo == FP8_GEMM_SKINNY && M > 64) return FP8_ERR_UNSUPPORTED;

  if (M == 0 || N == 0) return FP8_OK;
  if (!out) return FP8_ERR_NULL;
  if (!aligned(out, 16)) return FP8_ERR_ALIGN;
  const int64_t out_bytes = M * N * (out_dt == FP8_DT_F32 ? 4 : 2);
  if (K == 0) return hip_status(launch_fill_zero(out, out_bytes, stream));
  const fp8_status_t so = check_operands(p);
  if (so != FP8_OK) return so;
  p.out = out;
  const int path = accum == FP8_ACCUM_NATIVE ? PATH_FAST : PATH_EXACT;
  const bool skinny = (algo == FP8_GEMM_SKINNY) || (algo == FP8_GEMM_AUTO && M <= 64);
  if (skinny) return hip_status(launch_gemm_skinny(p, (int)a_fmt, (int)b_fmt, mode, (int)out_dt, path, stream));
  return hip_status(launch_gemm_tiled(p, (int)a_fmt, (int)b_fmt, mode, (int)out_dt, path, stream));
}

fp8_status_t fp8_gemm_blockscaled_quant(const uint8_t* a, fp8_format_t a_fmt, fp8_granularity_t a_g,
                                        const void* a_scales, const uint8_t* b, fp8_format_t b_fmt,
                                        fp8_granularity_t b_g, const void* b_scales, int64_t M, int64_t N,
                                        int64_t K, fp8_format_t out_fmt, uint8_t* out_codes, float* out_scales,
                                        fp8_accum_t accum, hipStream_t stream) {
  if (!valid_fmt(out_fmt)) return FP8_ERR_ENUM;
  GemmArgs p;
  int mode = 0;
  const fp8_status_t st = gemm_common(a, a_fmt, a_g, a_scales, b, b_fmt, b_g, b_scales, M, N, K, accum, p, mode);
  if (st != FP8_OK) return st;
  if (N % 128) return FP8_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8_OK;
  if (!out_codes || !out_scales) return FP8_ERR_NULL;
  if (!aligned(out_codes, 16) || !aligned(out_scales, 4)) return FP8_ERR_ALIGN;
  const int odt = out_fmt == FP8_E4M3 ? ODT_Q_E4M3 : ODT_Q_E5M2;
  p.out = out_codes;
  p.out_scales = out_scales;
  if (K == 0) {
    // all-zero result: codes 0, and the scale of an all-zero tile is 1
    const hipError_t e = launch_fill_zero(out_codes, M * N, stream);
    if (e != hipSuccess) return FP8_ERR_HIP;
    return hip_status(launch_fill_f32(out_scales, M * (N / 128), 1.0f, stream));
  }
  const fp8_status_t so = check_operands(p);
  if (so != FP8_OK) return so;
  const int path = accum == FP8_ACCUM_NATIVE ? PATH_FAST : PATH_EXACT;
  return hip_status(launch_gemm_tiled(p, (int)a_fmt, (int)b_fmt, mode, odt, path, stream));
}

fp8_status_t fp8_gemm_blockscaled(const uint8_t* a, fp8_format_t a_fmt, fp8_granularity_t a_g,
                                  const void* a_scales, const uint8_t* b, fp8_format_t b_fmt,
                                  fp8_granularity_t b_g, const void* b_scales, int64_t M, int64_t N, int64_t K,
                                  void* out, fp8_dtype_t out_dt, hipStream_t stream) {
  return fp8_gemm_blockscaled_ex(a, a_fmt, a_g, a_scales, b, b_fmt, b_g, b_scales, M, N, K, out, out_dt,
                                 FP8_GEMM_AUTO, FP8_ACCUM_FP32, stream);
}

fp8_status_t fp8_kv_append(const void* x, fp8_dtype_t x_dt, int64_t tokens, int64_t heads, int64_t head_dim,
                           int64_t ld_x, const int64_t* slots, fp8_format_t fmt, fp8_kv_scale_t scale_kind,
                           const float* scales, uint8_t* cache, int64_t num_slots, hipStream_t stream) {
  if (!valid_dt(x_dt) || !valid_fmt(fmt) || !valid_kv_scale(scale_kind)) return FP8_ERR_ENUM;
  const int64_t L = kv_row(heads, head_dim);
  if (L < 0 || tokens < 0 || num_slots < 0) return FP8_ERR_SHAPE;
  if (tokens == 0 || L == 0) return FP8_OK;
  const int64_t x_elems = mul_checked(tokens, ld_x);
  if (ld_x < L || x_elems < 0 || x_elems > INT64_MAX / 4 || mul_checked(num_slots, L) < 0) return FP8_ERR_SHAPE;
  if (!x || !slots || !scales || !cache) return FP8_ERR_NULL;
  const int64_t esize = x_dt == FP8_DT_BF16 ? 2 : 4;
  if (!aligned(x, 16) || (ld_x * esize) % 16 != 0 || !aligned(slots, 8) || !aligned(scales, 4) ||
      !aligned(cache, 16))
    return FP8_ERR_ALIGN;
  return hip_status(launch_kv_append(x, (int)x_dt, ld_x, slots, tokens, (int)fmt, (int)scale_kind, scales,
                                     (int)head_dim, L, cache, num_slots, stream));
}

fp8_status_t fp8_kv_gather(const uint8_t* cache, int64_t num_slots, int64_t heads, int64_t head_dim,
                           const int64_t* slots, int64_t n, fp8_format_t fmt, fp8_kv_scale_t scale_kind,
                           const float* scales, void* out, fp8_dtype_t out_dt, hipStream_t stream) {
  if (!valid_dt(out_dt) || !valid_fmt(fmt) || !valid_kv_scale(scale_kind)) return FP8_ERR_ENUM;
  const int64_t L = kv_row(heads, head_dim);
  if (L < 0 || n < 0 || num_slots < 0) return FP8_ERR_SHAPE;
  if (n == 0 || L == 0) return FP8_OK;
  const int64_t out_elems = mul_checked(n, L);
  if (out_elems < 0 || out_elems > INT64_MAX / 4 || mul_checked(num_slots, L) < 0) return FP8_ERR_SHAPE;
  if (!slots || !scales || !out || (num_slots > 0 && !cache)) return FP8_ERR_NULL;
  if (!aligned(cache, 16) || !aligned(slots, 8) || !aligned(scales, 4) || !aligned(out, 16)) return FP8_ERR_ALIGN;
  return hip_status(launch_kv_gather(cache, num_slots, slots, n, (int)fmt, (int)scale_kind, scales, (int)head_dim, L,
                                     out, (int)out_dt, stream));
}

size_t fp4_quantize_workspace_bytes(int64_t rows, int64_t cols, fp4_scaling_t kind) {
  if (!valid_fp4(kind) || check_operand(rows, cols, FP8_GRAN_ROW) != FP8_OK) return 0;
  return kind == FP4_SCALE_NV ? sizeof(float) * (size_t)kFp4Partials : 0;
}

fp8_status_t fp4_quantize(const void* x, fp8_dtype_t x_dt, int64_t rows, int64_t cols, fp4_scaling_t kind,
                          uint8_t* q, uint8_t* block_scales, float* tensor_scale, void* workspace, size_t ws_bytes,
                          hipStream_t stream) {
  if (!valid_dt(x_dt) || !valid_fp4(kind)) return FP8_ERR_ENUM;
  const fp8_status_t sh = check_operand(rows, cols, FP8_GRAN_ROW);
  if (sh != FP8_OK) return sh;
  const int64_t total = rows * cols;
  if (kind == FP4_SCALE_NV) {
    if (!tensor_scale) return FP8_ERR_NULL;
    if (!aligned(tensor_scale, 4)) return FP8_ERR_ALIGN;
  }
  if (total == 0) {
    if (kind == FP4_SCALE_MX) return FP8_OK;
    return hip_status(launch_fp4_quantize(x, (int)x_dt, rows, cols, (int)kind, q, block_scales, tensor_scale,
                                          nullptr, stream));
  }
  if (!x || !q || !block_scales) return FP8_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 16)) return FP8_ERR_ALIGN;
  if (kind == FP4_SCALE_NV) {
    if (!workspace || ws_bytes < sizeof(float) * (size_t)kFp4Partials) return FP8_ERR_WORKSPACE;
    if (!aligned(workspace, 4)) return FP8_ERR_ALIGN;
  }
  return hip_status(launch_fp4_quantize(x, (int)x_dt, rows, cols, (int)kind, q, block_scales, tensor_scale,
                                        static_cast<float*>(workspace), stream));
}

fp8_status_t fp4_dequantize(const uint8_t* q, const uint8_t* block_scales, const float* tensor_scale,
                            int64_t rows, int64_t cols, fp4_scaling_t kind, void* y, fp8_dtype_t y_dt,
                            hipStream_t stream) {
  if (!valid_dt(y_dt) || !valid_fp4(kind)) return FP8_ERR_ENUM;
  const fp8_status_t sh = check_operand(rows, cols, FP8_GRAN_ROW);
  if (sh != FP8_OK) return sh;
  if (rows * cols == 0) return FP8_OK;
  if (!q || !block_scales || !y || (kind == FP4_SCALE_NV && !tensor_scale)) return FP8_ERR_NULL;
  if (!aligned(q, 16) || !aligned(y, 16) || (kind == FP4_SCALE_NV && !aligned(tensor_scale, 4)))
    return FP8_ERR_ALIGN;
  return hip_status(launch_fp4_dequantize(q, block_scales, tensor_scale, rows, cols, (int)kind, y, (int)y_dt,
                                          stream));
}

fp8_status_t fp4_gemm_blockscaled(const uint8_t* a, const uint8_t* a_scales, const float* a_tensor_scale,
                                  const uint8_t* b, const uint8_t* b_scales, const float* b_tensor_scale,
                                  int64_t M, int64_t N, int64_t K, fp4_scaling_t kind, void* out,
                                  fp8_dtype_t out_dt, hipStream_t stream) {
  if (!valid_fp4(kind) || !valid_dt(out_dt)) return FP8_ERR_ENUM;
  if (M < 0 || N < 0 || K < 0 || M % 16 != 0 || N % 16 != 0 || K % 256 != 0 || K > kMaxGemmK) return FP8_ERR_SHAPE;
  if (mul_checked(M, N) < 0 || mul_checked(M, K) < 0 || mul_checked(N, K) < 0) return FP8_ERR_SHAPE;
  if ((M / 128 + 1) * (N / 128 + 1) >= INT_MAX) return FP8_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8_OK;
  if (!out) return FP8_ERR_NULL;
  if (!aligned(out, 16)) return FP8_ERR_ALIGN;
  const size_t esize = out_dt == FP8_DT_F32 ? 4 : 2;
  if (K == 0) return hip_status(launch_fill_zero(out, M * N * (int64_t)esize, stream));
  if (!a || !b || !a_scales || !b_scales) return FP8_ERR_NULL;
  if (kind == FP4_SCALE_NV && (!a_tensor_scale || !b_tensor_scale)) return FP8_ERR_NULL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(a_scales, 4) || !aligned(b_scales, 4)) return FP8_ERR_ALIGN;
  if (kind == FP4_SCALE_NV && (!aligned(a_tensor_scale, 4) || !aligned(b_tensor_scale, 4))) return FP8_ERR_ALIGN;
  GemmArgs p = GemmArgs{};
  p.a = a;
  p.b = b;
  p.sa = a_scales;
  p.sb = b_scales;
  p.ta = a_tensor_scale;
  p.tb = b_tensor_scale;
  p.out = out;
  p.M = M;
  p.N = N;
  p.K = K;
  p.ldo = N;
  // decode shapes (M <= 64) stream the weights through the skinny kernel, as
  // the FP8 GEMM's automatic choice does
  const int mode = kind == FP4_SCALE_MX ? MODE_MX4 : MODE_NV4;
  if (M <= 64) return hip_status(launch_gemm_skinny_fp4(p, mode, (int)out_dt, stream));
  return hip_status(launch_gemm_fp4(p, mode, (int)out_dt, stream));
}

}  // extern "C"
