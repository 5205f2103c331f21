// Skinny block-scaled FP8 GEMM for decode shapes (M <= 64, many output
// columns): out[M, N] = sum_k decode(a[m,k]) sA * decode(b[n,k]) sB, with the
// same scale modes and matrix-core paths as the tiled kernel in gemm.hip.
//
// At decode shapes the work is bound by reading W once from HBM ("The FP8
// Family", section "Where FP8 is winning": decode gains from bandwidth alone;
// "FP8 Serving", section "What FP8 actually buys": tokens/s follows bytes
// read).  The kernel is organised around the W stream:
//
//  * Balance per compute unit.  A streaming read on gfx950 is limited per
//    compute unit (a unit sustains roughly 1/256 of the chip's read rate,
//    measured), so the kernel time is set by the unit with the most bytes.
//    The grid is a multiple of the CU count and workgroup i owns the R =
//    ceil(N / grid) consecutive W rows [i R, i R + R): every unit streams the
//    same number of bytes.  R need not be a multiple of the 16-row matrix-core
//    tile; lanes of rows past the workgroup's range read zeros through the
//    buffer descriptor (no memory traffic) and their columns are not stored.
//  * X reuse.  The S waves of a workgroup split K into contiguous ranges and
//    each wave computes all T = ceil(R / 16) column tiles of its range, so an
//    X fragment (from L2: X is small) is fetched once per workgroup and used
//    T times, and the extra traffic through the unit is |X| per workgroup.
//  * Each wave keeps two 128-K steps of loads in flight in statically named
//    register sets.  Steps past the wave's range load through an out-of-range
//    offset (zeros, no memory traffic) and are not computed, so there are no
//    data-dependent branches around loads and the compiler's waits count
//    exactly the loads of older steps.
//  * The S partial tiles are added in LDS at the end.
#include "gemm_common.h"

namespace fp8blk {

// Registers of one 128-K step.
template <int MODE, int MT, int T>
struct SkinnyStep {
  u32x4 b[T][2];       // W fragment pieces, per column tile
  u32x4 a[MT][2];      // X fragment pieces, per 16-row tile of X
  float sx[MT][4];     // promotion: X scales of the lane's 4 rows
  uint32_t eb[T];      // MX: W scale byte of the lane's 32-K block
  uint32_t ea[MT];     // MX: X scale byte
};

// R (W rows per workgroup) <= 16 * T <= 112, so a workgroup's rows touch at
// most two 128-row W scale blocks.
template <int AF, int BF, int MODE, int ODT, int PATH, int MT, int T, int S>
__device__ __forceinline__ void gemm_skinny_body(const GemmArgs& p, int R) {
  static_assert(16 * T <= 112, "a workgroup's rows must touch at most two 128-row scale blocks");
  __shared__ __attribute__((aligned(16))) float red[S][MT * T][64][4];
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t n0 = (int64_t)blockIdx.x * R;
  if (n0 >= N) return;  // whole workgroup: no barrier has been reached
  const int nkb = (int)(K / 128);
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), g = lane >> 4;
  const int kb0 = (int)((int64_t)w * nkb / S), kb1 = (int)((int64_t)(w + 1) * nkb / S);
  const int64_t rows = (N - n0) < R ? (N - n0) : R;

  // Byte offsets of the lane's two 16-byte pieces inside a 128-K step:
  // exact path, 32 consecutive bytes (one MX block) per lane; fast path, the
  // FP8 instruction's K order.
  const int o0 = PATH == PATH_EXACT ? 32 * g : 16 * g;
  const int o1 = PATH == PATH_EXACT ? 32 * g + 16 : 64 + 16 * g;
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.b + n0 * K), 0, (int)(rows * K), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.a), 0, (int)(M * K), kBufferFlags);
  const int lrow = (lane & 15) * (int)K;
  const int tile_stride = 16 * (int)K;

  const float* sxa = reinterpret_cast<const float*>(p.sa);
  const float* swb = reinterpret_cast<const float*>(p.sb);
  const uint8_t* eab = reinterpret_cast<const uint8_t*>(p.sa);
  const uint8_t* ebb = reinterpret_cast<const uint8_t*>(p.sb);
  const int64_t kq = K / 32;
  // Promotion: the W scale of a lane's column is one of two per-step values
  // (blocks blo and blo + 1, clamped to the last block).
  const int64_t blo = n0 / 128, nblk = (N + 127) / 128;
  const float* sw_lo = swb + blo * nkb;
  const float* sw_hi = swb + (blo + 1 < nblk ? blo + 1 : blo) * nkb;
  bool hi[T];
#pragma unroll
  for (int t = 0; t < T; ++t) hi[t] = (n0 + 16 * t + (lane & 15)) / 128 > blo;

  v4f acc[MT][T];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[mt][t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  auto load = [&](SkinnyStep<MODE, MT, T>& Rg, int k) {
    const bool valid = k < kb1;
    const int kc = valid ? k : kb1 - 1;                  // scales: any valid step
    const int kk = valid ? k * 128 : kOutOfRange;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      Rg.b[t][0] = buffer_load16(rw, lrow + t * tile_stride + kk + o0);
      Rg.b[t][1] = buffer_load16(rw, lrow + t * tile_stride + kk + o1);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      Rg.a[mt][0] = buffer_load16(rx, lrow + mt * tile_stride + kk + o0);
      Rg.a[mt][1] = buffer_load16(rx, lrow + mt * tile_stride + kk + o1);
    }
    if constexpr (MODE == MODE_PROMOTE) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int64_t row = mt * 16 + 4 * g + r;
          row = row < M ? row : M - 1;
          Rg.sx[mt][r] = sxa[row * nkb + kc];
        }
    }
    if constexpr (MODE == MODE_MX) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        int64_t n = n0 + 16 * t + (lane & 15);
        n = n < N ? n : N - 1;
        Rg.eb[t] = ebb[n * kq + kc * 4 + g];
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        int64_t row = mt * 16 + (lane & 15);
        row = row < M ? row : M - 1;
        Rg.ea[mt] = eab[row * kq + kc * 4 + g];
      }
    }
  };

  auto compute = [&](const SkinnyStep<MODE, MT, T>& Rg, int k) {
    float f_lo[MT][4], f_hi[MT][4];
    if constexpr (MODE == MODE_PROMOTE) {
      const float s_lo = sw_lo[k], s_hi = sw_hi[k];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f_lo[mt][r] = Rg.sx[mt][r] * s_lo;
          f_hi[mt][r] = Rg.sx[mt][r] * s_hi;
        }
    }
    if constexpr (PATH == PATH_FAST) {
      v8i fa[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) fa[mt] = join(Rg.a[mt][0], Rg.a[mt][1]);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const v8i fb = join(Rg.b[t][0], Rg.b[t][1]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if constexpr (MODE == MODE_PROMOTE) {
            const v4f pr = mfma_fp8<AF, BF>(fa[mt], fb, v4f{0.0f, 0.0f, 0.0f, 0.0f}, (int)kUnitScale, (int)kUnitScale);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[mt][t][r] = __builtin_fmaf(pr[r], hi[t] ? f_hi[mt][r] : f_lo[mt][r], acc[mt][t][r]);
          } else if constexpr (MODE == MODE_MX) {
            acc[mt][t] = mfma_fp8<AF, BF>(fa[mt], fb, acc[mt][t], (int)Rg.ea[mt], (int)Rg.eb[t]);
          } else {
            acc[mt][t] = mfma_fp8<AF, BF>(fa[mt], fb, acc[mt][t], (int)kUnitScale, (int)kUnitScale);
          }
        }
      }
    } else {
      // X expanded once per step and reused for every column tile.
      v8bf xa[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const float fsa = (MODE == MODE_MX) ? e8m0_to_f32(Rg.ea[mt]) : 1.0f;
        xa[mt][0] = cvt8<AF>(Rg.a[mt][0].x, Rg.a[mt][0].y, fsa);
        xa[mt][1] = cvt8<AF>(Rg.a[mt][0].z, Rg.a[mt][0].w, fsa);
        xa[mt][2] = cvt8<AF>(Rg.a[mt][1].x, Rg.a[mt][1].y, fsa);
        xa[mt][3] = cvt8<AF>(Rg.a[mt][1].z, Rg.a[mt][1].w, fsa);
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float fsb = (MODE == MODE_MX) ? e8m0_to_f32(Rg.eb[t]) : 1.0f;
        v8bf xb[4];
        xb[0] = cvt8<BF>(Rg.b[t][0].x, Rg.b[t][0].y, fsb);
        xb[1] = cvt8<BF>(Rg.b[t][0].z, Rg.b[t][0].w, fsb);
        xb[2] = cvt8<BF>(Rg.b[t][1].x, Rg.b[t][1].y, fsb);
        xb[3] = cvt8<BF>(Rg.b[t][1].z, Rg.b[t][1].w, fsb);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if constexpr (MODE == MODE_PROMOTE) {
            v4f pp = mfma_bf16(xa[mt][0], xb[0], v4f{0.0f, 0.0f, 0.0f, 0.0f});
            pp = mfma_bf16(xa[mt][1], xb[1], pp);
            pp = mfma_bf16(xa[mt][2], xb[2], pp);
            pp = mfma_bf16(xa[mt][3], xb[3], pp);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[mt][t][r] = __builtin_fmaf(pp[r], hi[t] ? f_hi[mt][r] : f_lo[mt][r], acc[mt][t][r]);
          } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) acc[mt][t] = mfma_bf16(xa[mt][s], xb[s], acc[mt][t]);
          }
        }
      }
    }
  };

  // Two register sets with static names (a runtime index would put them in
  // scratch memory).
  SkinnyStep<MODE, MT, T> r0, r1;
  if (kb0 < kb1) {
    load(r0, kb0);
    for (int k = kb0; k < kb1; k += 2) {
      load(r1, k + 1);
      compute(r0, k);
      load(r0, k + 2);
      if (k + 1 < kb1) compute(r1, k + 1);
    }
  }

  // Partial tiles of the S waves -> LDS -> one sum per output element.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < T; ++t)
      *reinterpret_cast<float4*>(&red[w][mt * T + t][lane][0]) =
          make_float4(acc[mt][t][0], acc[mt][t][1], acc[mt][t][2], acc[mt][t][3]);
  __syncthreads();
  for (int u = w; u < MT * T; u += S) {
    const int mt = u / T, t = u % T;
    const int64_t cl = 16 * t + (lane & 15);  // column inside the workgroup's range
    if (cl >= rows) continue;
    const int64_t col = n0 + cl;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = mt * 16 + 4 * g + r;
      float v = 0.0f;
#pragma unroll
      for (int s = 0; s < S; ++s) v += red[s][u][lane][r];
      if (row >= M) continue;
      if constexpr (MODE == MODE_EPILOGUE) v = v * (sxa[p.a_per_row ? row : 0] * swb[p.b_per_row ? col : 0]);
      store_out<ODT>(p.out, row * N + col, v);
    }
  }
}

// Literal launch bounds (a template-dependent bound leaves the host stubs
// undefined).
template <int AF, int BF, int MODE, int ODT, int PATH, int MT, int T>
__global__ __launch_bounds__(256) void k_gemm_skinny(GemmArgs p, int R) {
  gemm_skinny_body<AF, BF, MODE, ODT, PATH, MT, T, 4>(p, R);
}

// ---- dispatch ----------------------------------------------------------------
// Tiles per workgroup by M (registers stay bounded): M <= 16: up to 5 tiles
// (R <= 80 rows), M <= 32: 3 (R <= 48), M <= 64: 2 (R <= 32).  The grid is
// c * CUs workgroups with the smallest c that keeps R within that bound.
template <int AF, int BF, int MODE, int ODT, int PATH, int MT, int T>
static void skinny_launch(const GemmArgs& p, hipStream_t st) {
  const int64_t cus = num_cus();
  const int64_t c = (p.N + cus * 16 * T - 1) / (cus * 16 * T);
  const int64_t grid = c * cus;
  int R = (int)((p.N + grid - 1) / grid);
  if (R < 16) R = 16;  // at least one full tile per workgroup (small N)
  hipLaunchKernelGGL((k_gemm_skinny<AF, BF, MODE, ODT, PATH, MT, T>), dim3((unsigned)grid), dim3(256), 0, st, p, R);
}

template <int AF, int BF, int MODE, int ODT, int PATH>
static void skinny_mt(const GemmArgs& p, hipStream_t st) {
  const int64_t mt = (p.M + 15) / 16;
  if (mt <= 1) skinny_launch<AF, BF, MODE, ODT, PATH, 1, 5>(p, st);
  else if (mt <= 2) skinny_launch<AF, BF, MODE, ODT, PATH, 2, 3>(p, st);
  else skinny_launch<AF, BF, MODE, ODT, PATH, 4, 2>(p, st);
}

template <int AF, int BF, int MODE, int ODT>
static void skinny_path(const GemmArgs& p, int path, hipStream_t st) {
  if (path == PATH_FAST) skinny_mt<AF, BF, MODE, ODT, PATH_FAST>(p, st);
  else skinny_mt<AF, BF, MODE, ODT, PATH_EXACT>(p, st);
}

template <int AF, int BF, int MODE>
static void skinny_odt(const GemmArgs& p, int odt, int path, hipStream_t st) {
  if (odt == DT_F32) skinny_path<AF, BF, MODE, DT_F32>(p, path, st);
  else skinny_path<AF, BF, MODE, DT_BF16>(p, path, st);
}

template <int AF, int BF>
static void skinny_mode(const GemmArgs& p, int mode, int odt, int path, hipStream_t st) {
  if (mode == MODE_EPILOGUE) skinny_odt<AF, BF, MODE_EPILOGUE>(p, odt, path, st);
  else if (mode == MODE_PROMOTE) skinny_odt<AF, BF, MODE_PROMOTE>(p, odt, path, st);
  else skinny_odt<AF, BF, MODE_MX>(p, odt, path, st);
}

hipError_t launch_gemm_skinny(const GemmArgs& p, int afmt, int bfmt, int mode, int odt, int path, hipStream_t st) {
  if (afmt == FMT_E4M3 && bfmt == FMT_E4M3) skinny_mode<FMT_E4M3, FMT_E4M3>(p, mode, odt, path, st);
  else if (afmt == FMT_E4M3) skinny_mode<FMT_E4M3, FMT_E5M2>(p, mode, odt, path, st);
  else if (bfmt == FMT_E4M3) skinny_mode<FMT_E5M2, FMT_E4M3>(p, mode, odt, path, st);
  else skinny_mode<FMT_E5M2, FMT_E5M2>(p, mode, odt, path, st);
  return hipGetLastError();
}

}  // namespace fp8blk
