// Device helpers shared by the gfx950 kernels of libfp8blk: FP8 encode/decode
// through the CDNA4 convert instructions, correctly rounded division by a
// per-group scale, and cross-lane max reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

enum { FMT_E4M3 = 0, FMT_E5M2 = 1 };
enum { DT_F32 = 0, DT_BF16 = 1 };
enum { G_TENSOR = 0, G_ROW = 1, G_TILE = 2, G_BLOCK = 3, G_MX = 4 };

// Largest finite value of each format: E4M3 1.75 * 2^8, E5M2 1.75 * 2^15.
template <int FMT> struct Fp8Limits;
template <> struct Fp8Limits<FMT_E4M3> { static constexpr float vmax = 448.0f;   static constexpr int emax = 8;  };
template <> struct Fp8Limits<FMT_E5M2> { static constexpr float vmax = 57344.0f; static constexpr int emax = 15; };

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Saturating round-to-nearest-even of four finite fp32 values to FP8 codes,
// packed so that element i lands in byte i.  The convert instruction rounds to
// nearest even; finite overflow is clamped beforehand with med3 (E4M3 has no
// Inf code, and values at or beyond the last rounding midpoint must map to Vmax).
template <int FMT>
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d) {
  constexpr float V = Fp8Limits<FMT>::vmax;
  a = __builtin_amdgcn_fmed3f(a, -V, V);
  b = __builtin_amdgcn_fmed3f(b, -V, V);
  c = __builtin_amdgcn_fmed3f(c, -V, V);
  d = __builtin_amdgcn_fmed3f(d, -V, V);
  int w;
  if constexpr (FMT == FMT_E4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return (uint32_t)w;
}

// Exact decode of the codes in bytes (2*hi, 2*hi+1) of w.
template <int FMT>
__device__ __forceinline__ v2f decode2(uint32_t w, bool hi) {
  if constexpr (FMT == FMT_E4M3) {
    return hi ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  } else {
    return hi ? __builtin_amdgcn_cvt_pk_f32_bf8(w, true) : __builtin_amdgcn_cvt_pk_f32_bf8(w, false);
  }
}

// RN32(x / s) for s > 2^-64 given y = RN32(1 / s).
// q0 = RN(x*y) is within a couple of ulps of x/s; one Newton correction with
// the FMA remainder makes it faithful, and a second one then yields the
// correctly rounded quotient (Markstein's theorem: y within half an ulp of 1/s
// and a faithful q give RN(q + (x - s q) y) = RN(x / s); P. Markstein, IBM J.
// Res. Dev. 34(1), 1990).  The remainder is formed as s*q - x and subtracted,
// which keeps the sign of zero quotients (x = -0 gives -0).
__device__ __forceinline__ float div_by_scale(float x, float s, float y) {
  float q = x * y;
  float r = __builtin_fmaf(s, q, -x);
  q = __builtin_fmaf(-r, y, q);
  r = __builtin_fmaf(s, q, -x);
  q = __builtin_fmaf(-r, y, q);
  return q;
}

// fp32 scale of a group: s = RN32(amax / Vmax), 1 when that is 0.  Plain '/'
// is the correctly rounded IEEE division in HIP device code.
template <int FMT>
__device__ __forceinline__ float group_scale(float amax) {
  float s = amax / Fp8Limits<FMT>::vmax;
  return s == 0.0f ? 1.0f : s;
}

// UE8M0 exponent: smallest e with amax <= Vmax * 2^e, clamped to [-127, 127];
// -127 for amax == 0.  amax = 1.f * 2^E; Vmax = 1.75 * 2^emax, so
// e = E - emax when 1.f <= 1.75 and E - emax + 1 otherwise.
template <int FMT>
__device__ __forceinline__ int mx_exponent(float amax) {
  uint32_t b = __float_as_uint(amax);
  int E;
  uint32_t frac;
  if ((b >> 23) == 0) {                 // zero or subnormal: normalise
    if (b == 0) return -127;
    int lz = __clz(b) - 8;              // shift to put the leading one at bit 23
    frac = (b << lz) & 0x7fffffu;
    E = -126 - lz;
  } else {
    frac = b & 0x7fffffu;
    E = (int)(b >> 23) - 127;
  }
  int e = (frac <= 0x600000u) ? E - Fp8Limits<FMT>::emax : E - Fp8Limits<FMT>::emax + 1;
  e = e < -127 ? -127 : e;
  e = e > 127 ? 127 : e;
  return e;
}

template <int N>
__device__ __forceinline__ float local_amax(const float* v) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) m = fmaxf(m, fabsf(v[i]));
  return m;
}

// Encode N (multiple of 4) values with the fp32 scale s into N/4 packed words.
template <int FMT, int N>
__device__ __forceinline__ void encode_scaled(const float* v, float s, uint32_t* out) {
  if (__builtin_expect(s >= 0x1p-64f, 1)) {
    const float y = 1.0f / s;
#pragma unroll
    for (int j = 0; j < N / 4; ++j)
      out[j] = encode4<FMT>(div_by_scale(v[4 * j], s, y), div_by_scale(v[4 * j + 1], s, y),
                            div_by_scale(v[4 * j + 2], s, y), div_by_scale(v[4 * j + 3], s, y));
  } else {
    // Tiny scale: scale x and s by 2^64 (exact) so that the quotient's
    // Newton steps stay in the normal range; the quotient is unchanged.
    const float s2 = s * 0x1p64f;
    const float y = 1.0f / s2;
#pragma unroll
    for (int j = 0; j < N / 4; ++j)
      out[j] = encode4<FMT>(div_by_scale(v[4 * j] * 0x1p64f, s2, y), div_by_scale(v[4 * j + 1] * 0x1p64f, s2, y),
                            div_by_scale(v[4 * j + 2] * 0x1p64f, s2, y), div_by_scale(v[4 * j + 3] * 0x1p64f, s2, y));
  }
}

// ---- cross-lane max (values are >= 0) --------------------------------------
// DPP row controls: quad_perm [1,0,3,2] (0xB1), [2,3,0,1] (0x4E),
// row_half_mirror (0x141), row_mirror (0x140).
template <int CTRL>
__device__ __forceinline__ float max_dpp(float v) {
  int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false);
  return fmaxf(v, __int_as_float(o));
}

// Max over aligned groups of LANES consecutive lanes (LANES in {1,2,4,8,16}).
template <int LANES>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (LANES >= 2) v = max_dpp<0xB1>(v);
  if constexpr (LANES >= 4) v = max_dpp<0x4E>(v);
  if constexpr (LANES >= 8) v = max_dpp<0x141>(v);
  if constexpr (LANES >= 16) v = max_dpp<0x140>(v);
  return v;
}

// Max over the whole 64-lane wave, result in every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = group_max<16>(v);
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// Max over the workgroup (blockDim.x a multiple of 64, at most 1024 threads),
// result in every thread.  `red` is LDS scratch of at least 16 floats.
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nw; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// Max of p[0..n) over one wave, eight independent loads in flight per lane
// (values >= 0 or NaN; fmaxf skips NaN, an empty input gives 0); result in
// every lane.
__device__ __forceinline__ float wave_max_of(const float* __restrict__ p, int64_t n) {
  const int lane = threadIdx.x & 63;
  float m[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) m[u] = 0.0f;
  int64_t i = lane;
  for (; i + 7 * 64 < n; i += 8 * 64) {
#pragma unroll
    for (int u = 0; u < 8; ++u) m[u] = fmaxf(m[u], p[i + u * 64]);
  }
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (i + u * 64 < n) m[u] = fmaxf(m[u], p[i + u * 64]);
  return wave_max(fmaxf(fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3])), fmaxf(fmaxf(m[4], m[5]), fmaxf(m[6], m[7]))));
}

// Max of p[0..n) over the workgroup (values >= 0 or NaN; fmaxf skips NaN, so
// an all-NaN or empty input gives 0), result in every thread.  Each thread
// keeps eight independent loads in flight: a loop with one load per trip
// waits a memory latency per element it visits.
__device__ __forceinline__ float block_max_of(const float* __restrict__ p, int64_t n, float* red) {
  const int64_t T = blockDim.x;
  float m[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) m[u] = 0.0f;
  int64_t i = threadIdx.x;
  for (; i + 7 * T < n; i += 8 * T) {
#pragma unroll
    for (int u = 0; u < 8; ++u) m[u] = fmaxf(m[u], p[i + u * T]);
  }
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (i + u * T < n) m[u] = fmaxf(m[u], p[i + u * T]);
  const float r = fmaxf(fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3])), fmaxf(fmaxf(m[4], m[5]), fmaxf(m[6], m[7])));
  return block_max(r, red);
}

}  // namespace fp8blk
