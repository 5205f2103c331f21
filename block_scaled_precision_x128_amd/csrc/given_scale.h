// Division by a scale that is given rather than taken from the data being
// encoded (delayed scaling, static KV-cache scales).  With current scaling
// |x / s| never exceeds Vmax by more than a rounding, but a given scale can be
// far below the data (the quotient then leaves the fp32 range) or far above
// it; the quantize formula still clips the real quotient to +-Vmax ("The FP8
// Family", quantize formula under "Scaling is what makes FP8 usable").
#pragma once

#include "device_common.h"

namespace fp8blk {

// Division constants of one positive scale s (s may be subnormal or +Inf):
//   x' = clamp(x, -bound, bound) * pre,  RN32(x / s) = RN32(x' / sd)
// bound = s * 2^17: any |x| beyond it has |x / s| > 2^17 > Vmax (both
// formats), so clamping changes no code but keeps the quotient finite.
// pre, sd: for s < 2^-64 both sides are scaled up by 2^64, for s > 2^64
// down by 2^64 (exactly, or the quotient is below 2^-126 and encodes to a
// signed zero either way), so that y = RN32(1 / sd) is a normal number and
// div_by_scale's Newton correction is exact; s = Inf gives signed zeros.
struct GivenScale {
  float sd, y, pre, bound;
};

__device__ __forceinline__ GivenScale given_scale(float s) {
  GivenScale g;
  g.bound = s * 0x1p17f;
  if (s < 0x1p-64f) {
    g.pre = 0x1p64f;
    g.sd = s * 0x1p64f;
  } else if (s > 0x1p64f) {
    const bool inf = __builtin_isinf(s);
    g.pre = inf ? 0.0f : 0x1p-64f;
    g.sd = inf ? 1.0f : s * 0x1p-64f;
  } else {
    g.pre = 1.0f;
    g.sd = s;
  }
  g.y = 1.0f / g.sd;
  return g;
}

__device__ __forceinline__ float quot_given(float x, const GivenScale& g) {
  x = __builtin_amdgcn_fmed3f(x, -g.bound, g.bound) * g.pre;
  return div_by_scale(x, g.sd, g.y);
}

// N (multiple of 4) values, one scale, into N/4 packed code words.
template <int FMT, int N>
__device__ __forceinline__ void encode_given(const float* v, const GivenScale& g, uint32_t* out) {
#pragma unroll
  for (int j = 0; j < N / 4; ++j)
    out[j] = encode4<FMT>(quot_given(v[4 * j], g), quot_given(v[4 * j + 1], g), quot_given(v[4 * j + 2], g),
                          quot_given(v[4 * j + 3], g));
}

}  // namespace fp8blk
