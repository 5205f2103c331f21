// FP4 (E2M1) quantization with two-level microscaling for gfx950: MXFP4
// (32 elements per UE8M0 scale) and NVFP4 (16 elements per E4M3 microscale,
// one fp32 scale per tensor), and the matching dequantization.
// ("Illustrated GPU kernels, Part 8", section "Low precision: FP8, FP4, and
// microscaling": the OCP MX block of 32 with a power-of-two scale, and NVFP4's
// blocks of 16 with an E4M3 microscale plus a tensor scale that keeps the
// microscales inside E4M3's range.)
//
// E2M1: 1 sign, 2 exponent, 1 mantissa bit, bias 1, magnitudes 0, 0.5, 1,
// 1.5, 2, 3, 4, 6, no Inf or NaN.  Two codes per byte, element 2i in the low
// nibble.  A thread handles 8 consecutive elements: one 16-byte bf16 load (two
// for fp32) and one 4-byte store of codes, contiguous across the wave; a scale
// block is 4 (MX) or 2 (NV) neighbouring lanes, whose amax is a DPP max.
#include "device_common.h"
#include "fp4.h"
#include "given_scale.h"

namespace fp8blk {

template <int DT>
__device__ __forceinline__ void fp4_load8(const void* __restrict__ x, int64_t e0, float* v) {
  if constexpr (DT == DT_BF16) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + e0);
    v[0] = bf16lo(w.x); v[1] = bf16hi(w.x); v[2] = bf16lo(w.y); v[3] = bf16hi(w.y);
    v[4] = bf16lo(w.z); v[5] = bf16hi(w.z); v[6] = bf16lo(w.w); v[7] = bf16hi(w.w);
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + e0);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Eight finite fp32 values to eight E2M1 codes, value i in nibble i (the low
// nibble of byte i/2 for even i): the hardware convert, with a unit scale,
// rounds to the nearest code with ties to the even one, saturates at 6 and
// keeps the sign (negative values that round to zero give -0, code 8).
__device__ __forceinline__ uint32_t e2m1_pack8(const float* q) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[0], q[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[4], q[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[6], q[7], 1.0f, 3);
  return w;
}

// Smallest e with amax <= 6 * 2^e, clamped to [-127, 127]; -127 for 0.
// amax = 1.f * 2^E and 6 = 1.5 * 2^2, so e = E - 2 when 1.f <= 1.5, else E - 1.
__device__ __forceinline__ int e2m1_mx_exponent(float amax) {
  const uint32_t b = __float_as_uint(amax);
  if (b == 0) return -127;
  int E;
  uint32_t frac;
  if ((b >> 23) == 0) {                  // subnormal: normalise
    const int lz = __clz(b) - 8;
    frac = (b << lz) & 0x7fffffu;
    E = -126 - lz;
  } else {
    frac = b & 0x7fffffu;
    E = (int)(b >> 23) - 127;
  }
  int e = frac <= 0x400000u ? E - 2 : E - 1;
  e = e < -127 ? -127 : e;
  return e > 127 ? 127 : e;
}

// MXFP4: chunk idx = elements [8 idx, 8 idx + 8); a 32-element block is 4 lanes.
template <int DT>
__global__ __launch_bounds__(256) void k_fp4_quant_mx(const void* __restrict__ x, uint8_t* __restrict__ q,
                                                       uint8_t* __restrict__ bs, int64_t nch) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= nch) return;   // nch % 4 == 0: a block's 4 lanes leave together
  float v[8];
  fp4_load8<DT>(x, 8 * idx, v);
  const float m = group_max<4>(local_amax<8>(v));
  const int e = e2m1_mx_exponent(m);
  float sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = __builtin_amdgcn_ldexpf(v[i], -e);   // exact: a power of two
  *reinterpret_cast<uint32_t*>(q + 4 * idx) = e2m1_pack8(sv);
  if ((idx & 3) == 0) bs[idx >> 2] = (uint8_t)(e + 127);
}

// NVFP4, pass 1: partial maxima of |x|.
template <int DT>
__global__ __launch_bounds__(256) void k_fp4_amax_partial(const void* __restrict__ x, int64_t nch,
                                                           float* __restrict__ partial) {
  __shared__ float red[16];
  float m = 0.0f;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < nch; idx += (int64_t)gridDim.x * 256) {
    float v[8];
    fp4_load8<DT>(x, 8 * idx, v);
    m = fmaxf(m, local_amax<8>(v));
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// NVFP4, pass 2: the tensor scale from the partial maxima, then per 16
// elements (2 lanes) the E4M3 microscale and the codes:
//   s_t = RN32(amax / 2688) (1 when 0); t = RN32(6 s_t); u = RN32(amax_b / t)
//   m = E4M3(u) (RNE, saturating); S = RN32(m s_t); codes = E2M1(RN32(x / S)),
//   signed zeros when S == 0.
template <int DT>
__global__ __launch_bounds__(256) void k_fp4_quant_nv(const void* __restrict__ x, uint8_t* __restrict__ q,
                                                       uint8_t* __restrict__ ms, float* __restrict__ ts,
                                                       int64_t nch, const float* __restrict__ partial,
                                                       int npartial) {
  __shared__ float red[16];
  const float mt = block_max_of(partial, npartial, red);
  float st = mt / 2688.0f;   // correctly rounded
  st = st == 0.0f ? 1.0f : st;
  if (blockIdx.x == 0 && threadIdx.x == 0) ts[0] = st;
  const float t = st * 6.0f;
  // nch is even and the stride is even: both lanes of a block run the same trips
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < nch; idx += (int64_t)gridDim.x * 256) {
    float v[8];
    fp4_load8<DT>(x, 8 * idx, v);
    const float mb = group_max<2>(local_amax<8>(v));
    const float u = mb / t;
    const uint32_t mcode = encode4<FMT_E4M3>(u, 0.0f, 0.0f, 0.0f) & 0xffu;
    const float S = decode2<FMT_E4M3>(mcode, false).x * st;
    uint32_t w = 0;
    if (S != 0.0f) {
      const GivenScale g = given_scale(S);
      float qv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[i] = quot_given(v[i], g);
      w = e2m1_pack8(qv);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w |= ((__float_as_uint(v[i]) >> 28) & 8u) << (4 * i);
    }
    *reinterpret_cast<uint32_t*>(q + 4 * idx) = w;
    if ((idx & 1) == 0) ms[idx >> 1] = (uint8_t)mcode;
  }
}

__device__ __forceinline__ uint32_t fp4_pack_bf16(float a, float b) {
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// Dequantize: E elements per thread (8 for bf16 output, 4 for fp32), one
// 16-byte store contiguous across the wave.  MX: decode(q) * 2^e (scale byte
// 255 reads as NaN); NV: RN32(decode(q) * S), S = RN32(m * s_t).  The codes
// decode exactly (scale 1 in the convert).
template <int KIND, int ODT>
__global__ __launch_bounds__(256) void k_fp4_dequant(const uint8_t* __restrict__ q, const uint8_t* __restrict__ bs,
                                                      const float* __restrict__ ts, int64_t total,
                                                      void* __restrict__ y) {
  constexpr int E = ODT == DT_F32 ? 4 : 8;
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * E;
  if (e0 >= total) return;
  uint32_t w;
  if constexpr (E == 8) w = *reinterpret_cast<const uint32_t*>(q + e0 / 2);
  else w = *reinterpret_cast<const uint16_t*>(q + e0 / 2);
  float v[E];
  {
    const v2f p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const v2f p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    v[0] = p0.x; v[1] = p0.y; v[2] = p1.x; v[3] = p1.y;
  }
  if constexpr (E == 8) {
    const v2f p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const v2f p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    v[4] = p2.x; v[5] = p2.y; v[6] = p3.x; v[7] = p3.y;
  }
  if constexpr (KIND == FP4_MX) {
    const uint32_t b = bs[e0 / 32];
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = b == 255u ? __builtin_nanf("") : __builtin_amdgcn_ldexpf(v[i], (int)b - 127);
  } else {
    const float S = decode2<FMT_E4M3>(bs[e0 / 16], false).x * ts[0];
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] *= S;
  }
  if constexpr (ODT == DT_F32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + e0) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(y) + e0) =
        u32x4{fp4_pack_bf16(v[0], v[1]), fp4_pack_bf16(v[2], v[3]), fp4_pack_bf16(v[4], v[5]),
              fp4_pack_bf16(v[6], v[7])};
  }
}

template <int DT>
static void fp4_quantize_t(const void* x, int64_t total, int kind, uint8_t* q, uint8_t* bs, float* ts, float* ws,
                           hipStream_t st) {
  const int64_t nch = total / 8;
  if (kind == FP4_MX) {
    hipLaunchKernelGGL((k_fp4_quant_mx<DT>), dim3((unsigned)((nch + 255) / 256)), dim3(256), 0, st, x, q, bs, nch);
    return;
  }
  int64_t p = (nch + 1023) / 1024;
  if (p > kFp4Partials) p = kFp4Partials;
  hipLaunchKernelGGL((k_fp4_amax_partial<DT>), dim3((unsigned)p), dim3(256), 0, st, x, nch, ws);
  int64_t p2 = (nch + 2047) / 2048;
  if (p2 > 2048) p2 = 2048;
  hipLaunchKernelGGL((k_fp4_quant_nv<DT>), dim3((unsigned)p2), dim3(256), 0, st, x, q, bs, ts, nch, ws, (int)p);
}

__global__ void k_fp4_unit_scale(float* ts) { ts[0] = 1.0f; }

hipError_t launch_fp4_quantize(const void* x, int dt, int64_t rows, int64_t cols, int kind, uint8_t* q,
                               uint8_t* bs, float* ts, float* ws, hipStream_t st) {
  const int64_t total = rows * cols;
  if (total == 0) {
    if (kind == FP4_NV) hipLaunchKernelGGL(k_fp4_unit_scale, dim3(1), dim3(1), 0, st, ts);
    return hipGetLastError();
  }
  if (dt == DT_BF16) fp4_quantize_t<DT_BF16>(x, total, kind, q, bs, ts, ws, st);
  else fp4_quantize_t<DT_F32>(x, total, kind, q, bs, ts, ws, st);
  return hipGetLastError();
}

hipError_t launch_fp4_dequantize(const uint8_t* q, const uint8_t* bs, const float* ts, int64_t rows, int64_t cols,
                                 int kind, void* y, int odt, hipStream_t st) {
  const int64_t total = rows * cols;
  if (total == 0) return hipSuccess;
  const int E = odt == DT_F32 ? 4 : 8;
  const dim3 grid((unsigned)((total / E + 255) / 256));
  if (kind == FP4_MX) {
    if (odt == DT_F32) hipLaunchKernelGGL((k_fp4_dequant<FP4_MX, DT_F32>), grid, dim3(256), 0, st, q, bs, ts, total, y);
    else hipLaunchKernelGGL((k_fp4_dequant<FP4_MX, DT_BF16>), grid, dim3(256), 0, st, q, bs, ts, total, y);
  } else {
    if (odt == DT_F32) hipLaunchKernelGGL((k_fp4_dequant<FP4_NV, DT_F32>), grid, dim3(256), 0, st, q, bs, ts, total, y);
    else hipLaunchKernelGGL((k_fp4_dequant<FP4_NV, DT_BF16>), grid, dim3(256), 0, st, q, bs, ts, total, y);
  }
  return hipGetLastError();
}

}  // namespace fp8blk
