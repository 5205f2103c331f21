// FP8 quantization kernels for gfx950: per-group amax, fp32 or UE8M0 scale,
// saturating round-to-nearest-even encode, packed stores.
//
// What is computed (pages "The FP8 Family", section "Scaling is what makes FP8
// usable"; "FP8 Mixed-Precision Serving", per-tensor and block-wise formulas;
// "Illustrated GPU kernels, Part 8", qdq listing and the OCP MX paragraph):
//   amax = max |x| over the group;  s = RN32(amax / Vmax)  (1 if that is 0)
//   code = sat_rne(RN32(x / s))                    fp32-scale modes
//   e = min{e : amax <= Vmax 2^e};  code = sat_rne(x * 2^-e)   MX32 mode
//
// Layout of work: every mode keeps a group's elements in registers between the
// amax and the encode, so the input is read from HBM once.
//   TILE_1x128  flat run of 128-element groups; 4 lanes x 32 elements per group
//   MX32        flat run of 32-element groups; 1 lane per group, no lane exchange
//   ROW         one workgroup per row (rows up to 256*8*CH elements in registers,
//               longer rows take a second pass that re-reads from L2)
//   BLOCK       one workgroup per 128x128 block, 64 elements per thread
//   TENSOR      amax partials per workgroup into the workspace, then a second
//               kernel reduces them and encodes; inputs up to 512 KiB in one
//               kernel whose every workgroup reduces the whole input itself
#include "device_common.h"
#include "given_scale.h"
#include "kernels.h"

namespace fp8blk {

// Per-tensor inputs up to this size are quantized in one launch (below).
constexpr int64_t kSmallTensorBytes = 512 * 1024;

// ---- loads of 8 / 32 consecutive elements as fp32 --------------------------
template <int DT>
__device__ __forceinline__ void load8(const void* __restrict__ x, int64_t e0, float* v) {
  if constexpr (DT == DT_BF16) {
    u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + e0);
    v[0] = bf16lo(w.x); v[1] = bf16hi(w.x); v[2] = bf16lo(w.y); v[3] = bf16hi(w.y);
    v[4] = bf16lo(w.z); v[5] = bf16hi(w.z); v[6] = bf16lo(w.w); v[7] = bf16hi(w.w);
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + e0);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <int DT, int E>
__device__ __forceinline__ void loadE(const void* __restrict__ x, int64_t e0, float* v) {
#pragma unroll
  for (int c = 0; c < E / 8; ++c) load8<DT>(x, e0 + 8 * c, v + 8 * c);
}

template <int FMT, int N>
__device__ __forceinline__ void encode_pow2(const float* v, int e, uint32_t* out) {
#pragma unroll
  for (int j = 0; j < N / 4; ++j)
    out[j] = encode4<FMT>(__builtin_amdgcn_ldexpf(v[4 * j], -e), __builtin_amdgcn_ldexpf(v[4 * j + 1], -e),
                          __builtin_amdgcn_ldexpf(v[4 * j + 2], -e), __builtin_amdgcn_ldexpf(v[4 * j + 3], -e));
}

// ---- flat groups: TILE_1x128 (G = 128) and MX32 (G = 32) -------------------
// Each lane owns 32 consecutive elements; G/32 consecutive lanes form a group.
template <int FMT, int DT, int G>
__global__ __launch_bounds__(256) void k_quant_flat(const void* __restrict__ x, uint8_t* __restrict__ q,
                                                     void* __restrict__ scales, int64_t total) {
  constexpr int E = 32, L = G / E;
  const int64_t lane_id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t e0 = lane_id * E;
  const bool valid = e0 < total;  // total is a multiple of G: groups are all-valid or all-invalid
  float v[E];
  if (valid) {
    loadE<DT, E>(x, e0, v);
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = 0.0f;
  }
  float m = group_max<L>(local_amax<E>(v));
  if (!valid) return;
  uint32_t out[E / 4];
  if constexpr (G == 32) {
    const int e = mx_exponent<FMT>(m);
    encode_pow2<FMT, E>(v, e, out);
    reinterpret_cast<uint8_t*>(scales)[e0 / 32] = (uint8_t)(e + 127);
  } else {
    const float s = group_scale<FMT>(m);
    encode_scaled<FMT, E>(v, s, out);
    if ((threadIdx.x & (L - 1)) == 0) reinterpret_cast<float*>(scales)[e0 / G] = s;
  }
  u32x4* dst = reinterpret_cast<u32x4*>(q + e0);
#pragma unroll
  for (int j = 0; j < E / 16; ++j) dst[j] = u32x4{out[4 * j], out[4 * j + 1], out[4 * j + 2], out[4 * j + 3]};
}

// ---- ROW: one workgroup per row ---------------------------------------------
template <int FMT, int DT, int CH>
__global__ __launch_bounds__(256) void k_quant_row(const void* __restrict__ x, uint8_t* __restrict__ q,
                                                    float* __restrict__ scales, int64_t cols) {
  __shared__ float red[16];
  const int64_t row = blockIdx.x;
  const int64_t base = row * cols;
  const int nch = (int)(cols / 8);
  float v[CH][8];
  float m = 0.0f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = threadIdx.x + 256 * c;
    if (idx < nch) {
      load8<DT>(x, base + 8 * (int64_t)idx, v[c]);
      m = fmaxf(m, local_amax<8>(v[c]));
    }
  }
  m = block_max(m, red);
  const float s = group_scale<FMT>(m);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = threadIdx.x + 256 * c;
    if (idx < nch) {
      uint32_t out[2];
      encode_scaled<FMT, 8>(v[c], s, out);
      *reinterpret_cast<u32x2*>(q + base + 8 * (int64_t)idx) = u32x2{out[0], out[1]};
    }
  }
  if (threadIdx.x == 0) scales[row] = s;
}

// Rows longer than the register budget: amax pass, then a re-reading encode pass.
template <int FMT, int DT>
__global__ __launch_bounds__(256) void k_quant_row_long(const void* __restrict__ x, uint8_t* __restrict__ q,
                                                         float* __restrict__ scales, int64_t cols) {
  __shared__ float red[16];
  const int64_t row = blockIdx.x;
  const int64_t base = row * cols;
  const int64_t nch = cols / 8;
  float m = 0.0f;
  for (int64_t idx = threadIdx.x; idx < nch; idx += 256) {
    float v[8];
    load8<DT>(x, base + 8 * idx, v);
    m = fmaxf(m, local_amax<8>(v));
  }
  m = block_max(m, red);
  const float s = group_scale<FMT>(m);
  for (int64_t idx = threadIdx.x; idx < nch; idx += 256) {
    float v[8];
    load8<DT>(x, base + 8 * idx, v);
    uint32_t out[2];
    encode_scaled<FMT, 8>(v, s, out);
    *reinterpret_cast<u32x2*>(q + base + 8 * idx) = u32x2{out[0], out[1]};
  }
  if (threadIdx.x == 0) scales[row] = s;
}

// ---- BLOCK_128x128: one workgroup per block ---------------------------------
// Thread t covers column chunk t%16 (8 elements) of rows t/16 + 16p, p = 0..7.
template <int FMT, int DT>
__global__ __launch_bounds__(256) void k_quant_block(const void* __restrict__ x, uint8_t* __restrict__ q,
                                                      float* __restrict__ scales, int64_t cols) {
  __shared__ float red[16];
  const int64_t ncb = cols / 128;
  const int64_t rb = blockIdx.x / ncb, cb = blockIdx.x % ncb;
  const int c8 = threadIdx.x & 15, r0 = threadIdx.x >> 4;
  float v[8][8];
  float m = 0.0f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int64_t row = rb * 128 + r0 + 16 * p;
    load8<DT>(x, row * cols + cb * 128 + c8 * 8, v[p]);
    m = fmaxf(m, local_amax<8>(v[p]));
  }
  m = block_max(m, red);
  const float s = group_scale<FMT>(m);
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int64_t row = rb * 128 + r0 + 16 * p;
    uint32_t out[2];
    encode_scaled<FMT, 8>(v[p], s, out);
    *reinterpret_cast<u32x2*>(q + row * cols + cb * 128 + c8 * 8) = u32x2{out[0], out[1]};
  }
  if (threadIdx.x == 0) scales[blockIdx.x] = s;
}

// ---- TENSOR: partial maxima, then reduce + encode ---------------------------
template <int DT>
__global__ __launch_bounds__(256) void k_amax_partial(const void* __restrict__ x, int64_t nch,
                                                       float* __restrict__ partial) {
  __shared__ float red[16];
  float m = 0.0f;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < nch; idx += (int64_t)gridDim.x * 256) {
    float v[8];
    load8<DT>(x, 8 * idx, v);
    m = fmaxf(m, local_amax<8>(v));
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

template <int FMT, int DT>
__global__ __launch_bounds__(256) void k_quant_tensor(const void* __restrict__ x, uint8_t* __restrict__ q,
                                                       float* __restrict__ scales, int64_t nch,
                                                       const float* __restrict__ partial, int npartial) {
  __shared__ float red[16];
  const float m = block_max_of(partial, npartial, red);
  const float s = group_scale<FMT>(m);
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < nch; idx += (int64_t)gridDim.x * 256) {
    float v[8];
    load8<DT>(x, 8 * idx, v);
    uint32_t out[2];
    encode_scaled<FMT, 8>(v, s, out);
    *reinterpret_cast<u32x2*>(q + 8 * idx) = u32x2{out[0], out[1]};
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) scales[0] = s;
}

// Small tensors in one launch: every workgroup reduces the amax of the whole
// tensor itself (after the first workgroup of an XCD touches the input, its
// reads hit that XCD's L2) and then encodes its own share of the chunks, so no
// partial maxima cross workgroups and no second launch waits for them.  The
// amax is a maximum, so the scale and codes are those of the two-kernel path.
// 1024 threads with eight 16-byte loads each in flight: the whole-tensor read
// is bound by the latency of a few rounds of loads, not by bandwidth.
template <int FMT, int DT>
__global__ __launch_bounds__(1024) void k_quant_tensor_small(const void* __restrict__ x, uint8_t* __restrict__ q,
                                                              float* __restrict__ scales, int64_t nch) {
  __shared__ float red[16];
  constexpr int T = 1024, U = DT == DT_BF16 ? 8 : 4;   // U chunks (U * 16 bytes) in flight per thread
  float mu[U];
#pragma unroll
  for (int u = 0; u < U; ++u) mu[u] = 0.0f;
  for (int64_t idx = threadIdx.x; idx < nch; idx += U * T) {
    float v[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (idx + u * T < nch) load8<DT>(x, 8 * (idx + u * T), v[u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (idx + u * T < nch) mu[u] = fmaxf(mu[u], local_amax<8>(v[u]));
  }
  float m = mu[0];
#pragma unroll
  for (int u = 1; u < U; ++u) m = fmaxf(m, mu[u]);
  m = block_max(m, red);
  const float s = group_scale<FMT>(m);
  for (int64_t i = (int64_t)blockIdx.x * T + threadIdx.x; i < nch; i += (int64_t)gridDim.x * T) {
    float v[8];
    load8<DT>(x, 8 * i, v);
    uint32_t out[2];
    encode_scaled<FMT, 8>(v, s, out);
    *reinterpret_cast<u32x2*>(q + 8 * i) = u32x2{out[0], out[1]};
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) scales[0] = s;
}

__global__ void k_fill_f32(float* p, float v) { *p = v; }

// ---- delayed scaling ----------------------------------------------------------
// ("FP8 Mixed-Precision Serving", section "Quantization Granularity and
// Scaling Topologies", delayed scaling.)  The scale comes from the amax
// history of earlier iterations, s = RN32(max(H) / (Vmax 2^-m)) = the inverse
// of rho = FP8max / (2^m max(H)); the tensor is encoded under it in one pass
// that also reduces its own amax, which then replaces history entry pos.
template <int FMT>
__global__ __launch_bounds__(256) void k_delayed_scale(const float* __restrict__ hist, int64_t len, int margin,
                                                        float* __restrict__ scale) {
  __shared__ float red[16];
  const float m = block_max_of(hist, len, red);  // NaN entries are skipped
  if (threadIdx.x == 0) {
    const float s = m / __builtin_amdgcn_ldexpf(Fp8Limits<FMT>::vmax, -margin);  // correctly rounded
    *scale = s == 0.0f ? 1.0f : s;
  }
}

// Encodes under the history's scale and reduces the tensor's amax per
// workgroup.  With a short history (FOLD) every wave derives the scale itself
// from the history, which saves the separate scale kernel's launch; the first
// wave writes it out.  Each thread keeps 4 chunks of loads in flight.
// partial[] holds one maximum per workgroup, so that the one-workgroup
// reduction after this kernel reads few values.
template <int FMT, int DT, bool FOLD>
__global__ __launch_bounds__(256) void k_quant_given_scale(const void* __restrict__ x, uint8_t* __restrict__ q,
                                                            float* __restrict__ scale, const float* __restrict__ hist,
                                                            int64_t len, int margin, int64_t nch,
                                                            float* __restrict__ partial) {
  float s;
  if constexpr (FOLD) {
    const float hm = wave_max_of(hist, len);  // NaN entries are skipped
    const float sv = hm / __builtin_amdgcn_ldexpf(Fp8Limits<FMT>::vmax, -margin);  // correctly rounded
    s = sv == 0.0f ? 1.0f : sv;
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale = s;
  } else {
    s = *scale;
  }
  const GivenScale gs = given_scale(s);
  float m = 0.0f;
  const int64_t G = (int64_t)gridDim.x * 256;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < nch; idx += 4 * G) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (idx + u * G < nch) load8<DT>(x, 8 * (idx + u * G), v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (idx + u * G < nch) {
        m = fmaxf(m, local_amax<8>(v[u]));
        uint32_t out[2];
        encode_given<FMT, 8>(v[u], gs, out);
        *reinterpret_cast<u32x2*>(q + 8 * (idx + u * G)) = u32x2{out[0], out[1]};
      }
    }
  }
  __shared__ float red[16];
  m = block_max(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

__global__ __launch_bounds__(256) void k_partials_to_slot(const float* __restrict__ partial, int npartial,
                                                           float* __restrict__ slot) {
  __shared__ float red[16];
  const float m = block_max_of(partial, npartial, red);
  if (threadIdx.x == 0) *slot = m;
}

template <int FMT, int DT>
static void quantize_delayed_t(const void* x, int64_t total, float* hist, int64_t len, int64_t pos, int margin,
                               uint8_t* q, float* scale, float* partial, hipStream_t st) {
  constexpr int64_t kFoldLen = 4096;   // history read by every workgroup up to this length
  if (total == 0 || len > kFoldLen)
    hipLaunchKernelGGL((k_delayed_scale<FMT>), dim3(1), dim3(256), 0, st, hist, len, margin, scale);
  if (total == 0) {
    hipLaunchKernelGGL(k_fill_f32, dim3(1), dim3(1), 0, st, hist + pos, 0.0f);
    return;
  }
  const int64_t nch = total / 8;
  int64_t p = (nch + 2047) / 2048;   // 8 chunks of 8 elements per thread
  if (p > kTensorPartials / 4) p = kTensorPartials / 4;   // grid-stride beyond that
  if (len > kFoldLen)
    hipLaunchKernelGGL((k_quant_given_scale<FMT, DT, false>), dim3((unsigned)p), dim3(256), 0, st, x, q, scale, hist,
                       len, margin, nch, partial);
  else
    hipLaunchKernelGGL((k_quant_given_scale<FMT, DT, true>), dim3((unsigned)p), dim3(256), 0, st, x, q, scale, hist,
                       len, margin, nch, partial);
  hipLaunchKernelGGL(k_partials_to_slot, dim3(1), dim3(256), 0, st, partial, (int)p, hist + pos);
}

hipError_t launch_quantize_delayed(const void* x, int dt, int64_t total, int fmt, float* hist, int64_t len,
                                   int64_t pos, int margin, uint8_t* q, float* scale, void* ws, hipStream_t st) {
  float* partial = reinterpret_cast<float*>(ws);
  if (fmt == FMT_E4M3) {
    if (dt == DT_BF16) quantize_delayed_t<FMT_E4M3, DT_BF16>(x, total, hist, len, pos, margin, q, scale, partial, st);
    else quantize_delayed_t<FMT_E4M3, DT_F32>(x, total, hist, len, pos, margin, q, scale, partial, st);
  } else {
    if (dt == DT_BF16) quantize_delayed_t<FMT_E5M2, DT_BF16>(x, total, hist, len, pos, margin, q, scale, partial, st);
    else quantize_delayed_t<FMT_E5M2, DT_F32>(x, total, hist, len, pos, margin, q, scale, partial, st);
  }
  return hipGetLastError();
}

// ---- unscaled cast, defined for every input ---------------------------------
template <int FMT>
__device__ __forceinline__ uint32_t cast_special_fix(float v, uint32_t code) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t mag = b & 0x7fffffffu;
  if (mag > 0x7f800000u) return 0x7Fu | sign;                              // NaN
  if (mag == 0x7f800000u) return (FMT == FMT_E4M3 ? 0x7Eu : 0x7Cu) | sign;  // +-Inf
  return code;
}

template <int FMT, int DT>
__global__ __launch_bounds__(256) void k_cast(const void* __restrict__ x, uint8_t* __restrict__ q, int64_t nch) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= nch) return;
  float v[8];
  load8<DT>(x, 8 * idx, v);
  uint32_t w[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint32_t c = encode4<FMT>(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) r |= cast_special_fix<FMT>(v[4 * j + i], (c >> (8 * i)) & 0xffu) << (8 * i);
    w[j] = r;
  }
  *reinterpret_cast<u32x2*>(q + 8 * idx) = u32x2{w[0], w[1]};
}

// ---- host launchers -----------------------------------------------------------
template <int FMT, int DT>
static hipError_t quantize_t(const void* x, int64_t rows, int64_t cols, int g, uint8_t* q, void* scales,
                             void* ws, hipStream_t st) {
  const int64_t total = rows * cols;
  switch (g) {
    case G_TILE:
    case G_MX: {
      if (total == 0) return hipSuccess;
      const int64_t lanes = total / 32;
      const int64_t blocks = (lanes + 255) / 256;
      if (g == G_TILE)
        hipLaunchKernelGGL((k_quant_flat<FMT, DT, 128>), dim3((unsigned)blocks), dim3(256), 0, st, x, q, scales, total);
      else
        hipLaunchKernelGGL((k_quant_flat<FMT, DT, 32>), dim3((unsigned)blocks), dim3(256), 0, st, x, q, scales, total);
      break;
    }
    case G_ROW: {
      if (total == 0) return hipSuccess;
      const int64_t nch = cols / 8;
      float* s = reinterpret_cast<float*>(scales);
      if (nch <= 256)
        hipLaunchKernelGGL((k_quant_row<FMT, DT, 1>), dim3((unsigned)rows), dim3(256), 0, st, x, q, s, cols);
      else if (nch <= 512)
        hipLaunchKernelGGL((k_quant_row<FMT, DT, 2>), dim3((unsigned)rows), dim3(256), 0, st, x, q, s, cols);
      else if (nch <= 1024)
        hipLaunchKernelGGL((k_quant_row<FMT, DT, 4>), dim3((unsigned)rows), dim3(256), 0, st, x, q, s, cols);
      else if (nch <= 2048)
        hipLaunchKernelGGL((k_quant_row<FMT, DT, 8>), dim3((unsigned)rows), dim3(256), 0, st, x, q, s, cols);
      else
        hipLaunchKernelGGL((k_quant_row_long<FMT, DT>), dim3((unsigned)rows), dim3(256), 0, st, x, q, s, cols);
      break;
    }
    case G_BLOCK: {
      if (total == 0) return hipSuccess;
      const int64_t nblk = (rows / 128) * (cols / 128);
      hipLaunchKernelGGL((k_quant_block<FMT, DT>), dim3((unsigned)nblk), dim3(256), 0, st, x, q,
                         reinterpret_cast<float*>(scales), cols);
      break;
    }
    case G_TENSOR: {
      float* s = reinterpret_cast<float*>(scales);
      if (total == 0) {
        hipLaunchKernelGGL(k_fill_f32, dim3(1), dim3(1), 0, st, s, 1.0f);
        break;
      }
      const int64_t nch = total / 8;
      if (total * (DT == DT_BF16 ? 2 : 4) <= kSmallTensorBytes) {
        // one workgroup per 2048 chunks, each reading the whole input once
        const int64_t gsm = (nch + 2047) / 2048;
        hipLaunchKernelGGL((k_quant_tensor_small<FMT, DT>), dim3((unsigned)gsm), dim3(1024), 0, st, x, q, s, nch);
        break;
      }
      int64_t p = (nch + 1023) / 1024;
      if (p > kTensorPartials) p = kTensorPartials;
      float* partial = reinterpret_cast<float*>(ws);
      hipLaunchKernelGGL((k_amax_partial<DT>), dim3((unsigned)p), dim3(256), 0, st, x, nch, partial);
      int64_t p2 = (nch + 2047) / 2048;
      if (p2 > 2048) p2 = 2048;
      hipLaunchKernelGGL((k_quant_tensor<FMT, DT>), dim3((unsigned)p2), dim3(256), 0, st, x, q, s, nch, partial,
                         (int)p);
      break;
    }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int dt, int64_t rows, int64_t cols, int fmt, int g, uint8_t* q,
                           void* scales, void* ws, hipStream_t st) {
  if (fmt == FMT_E4M3)
    return dt == DT_BF16 ? quantize_t<FMT_E4M3, DT_BF16>(x, rows, cols, g, q, scales, ws, st)
                         : quantize_t<FMT_E4M3, DT_F32>(x, rows, cols, g, q, scales, ws, st);
  return dt == DT_BF16 ? quantize_t<FMT_E5M2, DT_BF16>(x, rows, cols, g, q, scales, ws, st)
                       : quantize_t<FMT_E5M2, DT_F32>(x, rows, cols, g, q, scales, ws, st);
}

hipError_t launch_cast(const void* x, int dt, int64_t n, int fmt, uint8_t* q, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t nch = n / 8;
  const dim3 grid((unsigned)((nch + 255) / 256));
  if (fmt == FMT_E4M3) {
    if (dt == DT_BF16) hipLaunchKernelGGL((k_cast<FMT_E4M3, DT_BF16>), grid, dim3(256), 0, st, x, q, nch);
    else hipLaunchKernelGGL((k_cast<FMT_E4M3, DT_F32>), grid, dim3(256), 0, st, x, q, nch);
  } else {
    if (dt == DT_BF16) hipLaunchKernelGGL((k_cast<FMT_E5M2, DT_BF16>), grid, dim3(256), 0, st, x, q, nch);
    else hipLaunchKernelGGL((k_cast<FMT_E5M2, DT_F32>), grid, dim3(256), 0, st, x, q, nch);
  }
  return hipGetLastError();
}

}  // namespace fp8blk
