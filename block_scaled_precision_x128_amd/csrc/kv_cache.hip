// FP8 KV cache for gfx950: quantize on append, dequantize on read.
// ("FP8 Mixed-Precision Serving", section "FP8 KV Cache Architecture and
// Serving Latency": key and value states held as one-byte E4M3 codes, half the
// bytes of bf16, which is what decode reads every step; "FP8 Serving", the
// quality table and "Things to try": a per-tensor scale, a per-channel one for
// channel-structured outliers, E5M2 for range.)
//
// The cache is a pool of slots, each one token's L = heads * head_dim codes.
// A thread owns 16 elements of a row for all of the rows it visits (rows
// advance by a fixed row step), so per-head and per-channel scales, and the
// division constants of the append, are loaded and prepared once per thread
// rather than per element.  Both kernels are pure streams: 1 code byte plus 2
// (bf16) or 4 (fp32) bytes of values per element, and 8 bytes of slot index
// per row.
//   append: thread c owns elements [16c, 16c + 16): its 16 code bytes are one
//           store, and the stores of a wave cover a contiguous 1 KB.
//   read:   the 16 elements are P pieces of 16/P, at elements (16/P)(c + p L/16)
//           for p < P, so that every 16-byte store of the output (8 bf16 or 4
//           fp32 values) is contiguous across the wave.  Stores at a 32-byte
//           lane stride (16 contiguous elements per thread) measured 15-20%
//           slower on this write-heavy stream.
#include "device_common.h"
#include "gemm_common.h"  // num_cus()
#include "given_scale.h"
#include "kv_cache.h"

namespace fp8blk {

enum { KV_TENSOR = 0, KV_HEAD = 1, KV_CHANNEL = 2 };

template <int DT>
__device__ __forceinline__ void kv_load16(const void* __restrict__ x, int64_t e0, float* v) {
  if constexpr (DT == DT_BF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + e0);
    const u32x4 a = p[0], b = p[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = bf16lo(w[i]);
      v[2 * i + 1] = bf16hi(w[i]);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + e0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 a = p[i];
      v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
    }
  }
}

__device__ __forceinline__ uint32_t kv_pack_bf16(float a, float b) {
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

struct KvShape {
  int64_t rows;       // tokens to append / rows to read
  int64_t row_step;   // rows in flight per pass (grid rows)
  int64_t num_slots;  // slots in the pool
  int cpr;            // 16-element chunks per row (L / 16)
  int head_dim;
};

// cache[slots[r]] = codes of x[r] for every r with 0 <= slots[r] < num_slots.
template <int FMT, int DT, int SK>
__global__ __launch_bounds__(256) void k_kv_append(const void* __restrict__ x, int64_t ld_x,
                                                    const int64_t* __restrict__ slots,
                                                    const float* __restrict__ scales, KvShape sh,
                                                    uint8_t* __restrict__ cache) {
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t r = tid / sh.cpr;
  if (r >= sh.row_step) return;
  const int e0 = 16 * (int)(tid - r * sh.cpr);
  const int64_t L = (int64_t)sh.cpr * 16;
  constexpr int NS = SK == KV_CHANNEL ? 16 : 1;
  GivenScale g[NS];
  if constexpr (SK == KV_TENSOR) {
    g[0] = given_scale(scales[0]);
  } else if constexpr (SK == KV_HEAD) {
    g[0] = given_scale(scales[e0 / sh.head_dim]);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) g[i] = given_scale(scales[e0 + i]);
  }
  for (; r < sh.rows; r += sh.row_step) {
    const int64_t slot = slots[r];
    float v[16];
    kv_load16<DT>(x, r * ld_x + e0, v);
    if ((uint64_t)slot >= (uint64_t)sh.num_slots) continue;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const GivenScale* gj = g + (NS == 16 ? 4 * j : 0);
      const int st = NS == 16 ? 1 : 0;
      w[j] = encode4<FMT>(quot_given(v[4 * j], gj[0]), quot_given(v[4 * j + 1], gj[st]),
                          quot_given(v[4 * j + 2], gj[2 * st]), quot_given(v[4 * j + 3], gj[3 * st]));
    }
    *reinterpret_cast<u32x4*>(cache + slot * L + e0) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// out[r] = RN32(decode(cache[slots[r]]) * s), then bf16 (nearest even) when
// ODT is bf16; zeros for a slot outside the pool.  out is [rows, L].  Two rows
// per iteration: both slot loads, then both rows' code loads, are in flight
// together.
template <int FMT, int SK, int ODT>
__global__ __launch_bounds__(256) void k_kv_gather(const uint8_t* __restrict__ cache,
                                                    const int64_t* __restrict__ slots,
                                                    const float* __restrict__ scales, KvShape sh,
                                                    void* __restrict__ out) {
  constexpr int P = ODT == DT_F32 ? 4 : 2;   // pieces per thread
  constexpr int E = 16 / P;                  // elements per piece: one 16-byte output store
  constexpr int U = 2;                       // rows per iteration
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t r = tid / sh.cpr;
  if (r >= sh.row_step) return;
  const int c = (int)(tid - r * sh.cpr);
  const int64_t L = (int64_t)sh.cpr * 16;
  int ep[P];
#pragma unroll
  for (int p = 0; p < P; ++p) ep[p] = E * (c + p * sh.cpr);
  constexpr int NS = SK == KV_CHANNEL ? 16 : (SK == KV_HEAD ? P : 1);
  float s[NS];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    if constexpr (SK == KV_CHANNEL) {
#pragma unroll
      for (int i = 0; i < E; ++i) s[p * E + i] = scales[ep[p] + i];
    } else if constexpr (SK == KV_HEAD) {
      s[p] = scales[ep[p] / sh.head_dim];
    } else {
      if (p == 0) s[0] = scales[0];
    }
  }
  for (; r < sh.rows; r += U * sh.row_step) {
    int64_t slot[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t rr = r + u * sh.row_step;
      slot[u] = rr < sh.rows ? slots[rr] : -1;
    }
    uint32_t w[U][P][E / 4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = (uint64_t)slot[u] < (uint64_t)sh.num_slots;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        if constexpr (E == 8) {
          const u32x2 q = ok ? *reinterpret_cast<const u32x2*>(cache + slot[u] * L + ep[p]) : u32x2{0, 0};
          w[u][p][0] = q.x;
          w[u][p][1] = q.y;
        } else {
          w[u][p][0] = ok ? *reinterpret_cast<const uint32_t*>(cache + slot[u] * L + ep[p]) : 0u;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t rr = r + u * sh.row_step;
      if (rr >= sh.rows) break;
      const bool ok = (uint64_t)slot[u] < (uint64_t)sh.num_slots;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        float v[E];
#pragma unroll
        for (int i = 0; i < E / 4; ++i) {
          const v2f lo = decode2<FMT>(w[u][p][i], false), hi = decode2<FMT>(w[u][p][i], true);
          v[4 * i] = lo.x; v[4 * i + 1] = lo.y; v[4 * i + 2] = hi.x; v[4 * i + 3] = hi.y;
        }
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const float si = s[SK == KV_CHANNEL ? p * E + i : (SK == KV_HEAD ? p : 0)];
          v[i] = ok ? v[i] * si : 0.0f;
        }
        if constexpr (ODT == DT_F32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + rr * L + ep[p]) =
              make_float4(v[0], v[1], v[2], v[3]);
        } else {
          *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + rr * L + ep[p]) =
              u32x4{kv_pack_bf16(v[0], v[1]), kv_pack_bf16(v[2], v[3]), kv_pack_bf16(v[4], v[5]),
                    kv_pack_bf16(v[6], v[7])};
        }
      }
    }
  }
}

// Rows in flight: threads for 4 workgroups of 256 per CU (measured: more
// waves per CU slow these write-carrying streams down, fewer leave reads
// short of requests), but no more rows than there are.
static KvShape kv_shape(int64_t rows, int64_t num_slots, int64_t L, int head_dim) {
  KvShape sh;
  sh.rows = rows;
  sh.num_slots = num_slots;
  sh.cpr = (int)(L / 16);
  sh.head_dim = head_dim;
  const int64_t target = (int64_t)num_cus() * 4 * 256;
  const int64_t rs = (target + sh.cpr - 1) / sh.cpr;
  sh.row_step = rows < rs ? rows : rs;
  return sh;
}

static dim3 kv_grid(const KvShape& sh) { return dim3((unsigned)((sh.row_step * sh.cpr + 255) / 256)); }

template <int FMT, int DT>
static void kv_append_t(const void* x, int64_t ld_x, const int64_t* slots, int sk, const float* scales,
                        const KvShape& sh, uint8_t* cache, hipStream_t st) {
  const dim3 grid = kv_grid(sh);
  if (sk == KV_TENSOR)
    hipLaunchKernelGGL((k_kv_append<FMT, DT, KV_TENSOR>), grid, dim3(256), 0, st, x, ld_x, slots, scales, sh, cache);
  else if (sk == KV_HEAD)
    hipLaunchKernelGGL((k_kv_append<FMT, DT, KV_HEAD>), grid, dim3(256), 0, st, x, ld_x, slots, scales, sh, cache);
  else
    hipLaunchKernelGGL((k_kv_append<FMT, DT, KV_CHANNEL>), grid, dim3(256), 0, st, x, ld_x, slots, scales, sh,
                       cache);
}

hipError_t launch_kv_append(const void* x, int dt, int64_t ld_x, const int64_t* slots, int64_t tokens, int fmt,
                            int sk, const float* scales, int head_dim, int64_t L, uint8_t* cache, int64_t num_slots,
                            hipStream_t st) {
  if (tokens == 0 || L == 0) return hipSuccess;
  const KvShape sh = kv_shape(tokens, num_slots, L, head_dim);
  if (fmt == FMT_E4M3) {
    if (dt == DT_BF16) kv_append_t<FMT_E4M3, DT_BF16>(x, ld_x, slots, sk, scales, sh, cache, st);
    else kv_append_t<FMT_E4M3, DT_F32>(x, ld_x, slots, sk, scales, sh, cache, st);
  } else {
    if (dt == DT_BF16) kv_append_t<FMT_E5M2, DT_BF16>(x, ld_x, slots, sk, scales, sh, cache, st);
    else kv_append_t<FMT_E5M2, DT_F32>(x, ld_x, slots, sk, scales, sh, cache, st);
  }
  return hipGetLastError();
}

template <int FMT, int ODT>
static void kv_gather_t(const uint8_t* cache, const int64_t* slots, int sk, const float* scales, const KvShape& sh,
                        void* out, hipStream_t st) {
  const dim3 grid = kv_grid(sh);
  if (sk == KV_TENSOR)
    hipLaunchKernelGGL((k_kv_gather<FMT, KV_TENSOR, ODT>), grid, dim3(256), 0, st, cache, slots, scales, sh, out);
  else if (sk == KV_HEAD)
    hipLaunchKernelGGL((k_kv_gather<FMT, KV_HEAD, ODT>), grid, dim3(256), 0, st, cache, slots, scales, sh, out);
  else
    hipLaunchKernelGGL((k_kv_gather<FMT, KV_CHANNEL, ODT>), grid, dim3(256), 0, st, cache, slots, scales, sh, out);
}

hipError_t launch_kv_gather(const uint8_t* cache, int64_t num_slots, const int64_t* slots, int64_t n, int fmt, int sk,
                            const float* scales, int head_dim, int64_t L, void* out, int odt, hipStream_t st) {
  if (n == 0 || L == 0) return hipSuccess;
  const KvShape sh = kv_shape(n, num_slots, L, head_dim);
  if (fmt == FMT_E4M3) {
    if (odt == DT_BF16) kv_gather_t<FMT_E4M3, DT_BF16>(cache, slots, sk, scales, sh, out, st);
    else kv_gather_t<FMT_E4M3, DT_F32>(cache, slots, sk, scales, sh, out, st);
  } else {
    if (odt == DT_BF16) kv_gather_t<FMT_E5M2, DT_BF16>(cache, slots, sk, scales, sh, out, st);
    else kv_gather_t<FMT_E5M2, DT_F32>(cache, slots, sk, scales, sh, out, st);
  }
  return hipGetLastError();
}

}  // namespace fp8blk
