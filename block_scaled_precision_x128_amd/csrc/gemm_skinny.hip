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
//  * Full-line loads.  W and X reach LDS through loads that write LDS
//    directly, each instruction fetching 8 whole 128-byte rows (a load of the
//    matrix-core fragments straight into registers fetches 16 half rows per
//    instruction, and the unit's request rate, not its byte rate, then bounds
//    the stream).  Fragments are read back from LDS in the matrix-core
//    layout, through the same conflict-free chunk swizzle as the tiled kernel.
//  * Each wave owns two LDS stages: the loads of step k+1 are in flight while
//    step k is computed.  Steps past the wave's range load zeros (no memory
//    traffic) and are not computed, so every step issues the same loads and
//    a fixed s_waitcnt count leaves exactly one step's loads in flight.
//  * The S partial tiles are added in LDS at the end.
#include "gemm_common.h"

namespace fp8blk {

// LDS footprint of one wave's stage (bytes): W rows, X rows, then scales.
// A step is 128 bytes of every row: 128 K of FP8 codes, 256 K of FP4 codes.
// Scale words per step: MX one per row (4 UE8M0 bytes), MXFP4 two, NVFP4 four
// (16 E4M3 microscales, staged row by row: 16 bytes per row).  MODE_MX4_PAIRS
// stages the 16-byte aligned block of a row's scale bytes that holds the
// step's 8 (those of the step pair), also row by row.
template <int MODE, int MT, int T>
struct SkinnyStage {
  static constexpr int kW = 16 * T * 128;          // W tile rows (128 bytes each)
  static constexpr int kX = 16 * MT * 128;         // X tile rows
  static constexpr bool kRow16 = MODE == MODE_NV4 || MODE == MODE_MX4_PAIRS;
  static constexpr int kScaleLoads =
      MODE == MODE_PROMOTE ? 2 : (MODE == MODE_MX ? 3 : (MODE == MODE_MX4 ? 6 : (kRow16 ? 3 : 0)));
  // NVFP4 and MODE_MX4_PAIRS stage 16 scale bytes per row with one 16-byte load per 64 rows
  static constexpr int kScale = kScaleLoads * (kRow16 ? 1024 : 256);
  static constexpr int kBytes = kW + kX + kScale;
  // loads issued per step (every one is issued, out-of-range ones read zeros)
  static constexpr int kLoads = 2 * T + 2 * MT + kScaleLoads;
};

// R (W rows per workgroup) <= 16 * T <= 112, so a workgroup's rows touch at
// most two 128-row W scale blocks and their MX scale words fit two 64-lane loads.
template <int AF, int BF, int MODE, int ODT, int PATH, int MT, int T, int S, int NS>
__device__ __forceinline__ void gemm_skinny_body(const GemmArgs& p, int R) {
  static_assert(16 * T <= 112, "a workgroup's rows must touch at most two 128-row scale blocks");
  using St = SkinnyStage<MODE, MT, T>;
  static_assert(NS * St::kLoads <= 63, "loads in flight must fit the vmcnt counter");
  static_assert(MT * T * 64 * 16 <= NS * St::kBytes, "partial tiles must fit in the wave's stages");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[S][NS][St::kBytes];

  const int64_t M = p.M, N = p.N;
  constexpr bool PAIRS = MODE == MODE_MX4_PAIRS;
  constexpr bool MX4 = MODE == MODE_MX4 || PAIRS;
  constexpr bool FP4 = MX4 || MODE == MODE_NV4;
  static_assert(!MX4 || PATH == PATH_FAST, "MXFP4 runs on the FP4 matrix cores");
  static_assert(MODE != MODE_NV4 || PATH == PATH_EXACT, "NVFP4 runs on exact fp16 expansions");
  const int64_t K = FP4 ? p.K / 2 : p.K;   // bytes per operand row
  const int64_t n0 = (int64_t)blockIdx.x * R;
  if (n0 >= N) return;  // whole workgroup: no barrier has been reached
  const int nkb = (int)(K / 128);
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), g = lane >> 4;
  const int kb0 = (int)((int64_t)w * nkb / S), kb1 = (int)((int64_t)(w + 1) * nkb / S);
  const int64_t rows = (N - n0) < R ? (N - n0) : R;
  const int64_t kq = MODE == MODE_NV4 ? p.K / 16 : p.K / 32;   // scale bytes per row

  // Loads into LDS, 8 full 128-byte rows per instruction: lane q takes row
  // q/8 of its 8-row block and stored chunk q%8, i.e. logical chunk
  // (q%8) ^ lds_swz(row); lds_swz(8u + q/8) = (q/8) ^ (u & 1).
  const int q8 = lane >> 3;
  const int off_even = q8 * (int)K + (((lane & 7) ^ q8) << 4);
  const int off_odd = q8 * (int)K + (((lane & 7) ^ q8 ^ 1) << 4);
  auto rsrc = [&](const void* base, int64_t bytes) { return uniform_rsrc(base, bytes); };
  const uint8_t* wbase = p.b + n0 * K;
  const float* sxa = reinterpret_cast<const float*>(p.sa);
  const float* swb = reinterpret_cast<const float*>(p.sb);
  const int64_t blo = n0 / 128, nblk = (N + 127) / 128;
  // descriptors of the per-step scale loads
  __amdgpu_buffer_rsrc_t rs_sx = rsrc(p.sa, 0), rs_sw = rsrc(p.sb, 0), rs_ex = rsrc(p.sa, 0), rs_ew = rsrc(p.sb, 0);
  if constexpr (MODE == MODE_PROMOTE) {
    rs_sx = rsrc(sxa, M * nkb * 4);                                    // sA[m, kb], lanes m < M
    rs_sw = rsrc(swb + blo * nkb, ((blo + 1 < nblk) ? 2 : 1) * nkb * 4);  // sB[blo + l, kb], l < 2
  }
  if constexpr (MODE == MODE_MX || FP4) {
    rs_ex = rsrc(p.sa, M * kq);                                        // scale bytes of row m, step kb
    rs_ew = rsrc(reinterpret_cast<const uint8_t*>(p.sb) + n0 * kq, rows * kq);
  }

  auto issue = [&](int k, int stage) {
    const bool valid = k < kb1;
    const int kk = valid ? k * 128 : kOutOfRange;
    uint8_t* st = &lds[w][stage][0];
#pragma unroll
    for (int u = 0; u < 2 * T; ++u) {
      const int64_t left = rows - 8 * u;
      dma_to_lds<16>(rsrc(wbase + 8 * u * K, left * K), lds_addr(st + 8 * u * 128), off_add((u & 1) ? off_odd : off_even, kk));
    }
#pragma unroll
    for (int u = 0; u < 2 * MT; ++u) {
      const int64_t left = M - 8 * u;
      dma_to_lds<16>(rsrc(p.a + 8 * u * K, left * K), lds_addr(st + St::kW + 8 * u * 128),
                     off_add((u & 1) ? off_odd : off_even, kk));
    }
    uint8_t* sc = st + St::kW + St::kX;
    if constexpr (MODE == MODE_PROMOTE) {
      const int ks = valid ? k * 4 : kOutOfRange;
      dma_to_lds<4>(rs_sx, lds_addr(sc), off_add(lane * nkb * 4, ks));
      dma_to_lds<4>(rs_sw, lds_addr(sc + 256), off_add(lane * nkb * 4, ks));
    }
    if constexpr (MODE == MODE_MX) {
      const int ks = valid ? k * 4 : kOutOfRange;
      dma_to_lds<4>(rs_ex, lds_addr(sc), off_add(lane * (int)kq, ks));
      dma_to_lds<4>(rs_ew, lds_addr(sc + 256), off_add(lane * (int)kq, ks));
      dma_to_lds<4>(rs_ew, lds_addr(sc + 512), off_add((64 + lane) * (int)kq, ks));
    }
    if constexpr (MODE == MODE_MX4) {
      // word wd (UE8M0 bytes 4wd .. 4wd+3 of the step) of X rows at sc + 256 wd,
      // of W rows r < 128 at sc + 512 + 512 wd + 4 r
      const int ks = valid ? k * 8 : kOutOfRange;
#pragma unroll
      for (int wd = 0; wd < 2; ++wd) {
        dma_to_lds<4>(rs_ex, lds_addr(sc + 256 * wd), off_add(lane * (int)kq + 4 * wd, ks));
        dma_to_lds<4>(rs_ew, lds_addr(sc + 512 + 512 * wd), off_add(lane * (int)kq + 4 * wd, ks));
        dma_to_lds<4>(rs_ew, lds_addr(sc + 768 + 512 * wd), off_add((64 + lane) * (int)kq + 4 * wd, ks));
      }
    }
    if constexpr (MODE == MODE_NV4 || PAIRS) {
      // a row's 16 microscale bytes of the step (NVFP4), or the 16 scale
      // bytes of the step pair (MODE_MX4_PAIRS), in one 16-byte load (kq and
      // the offset are multiples of 16): X rows at sc + 16 r, W rows r < 128
      // at sc + 1024 + 16 r
      const int ks = valid ? (PAIRS ? (k & ~1) * 8 : k * 16) : kOutOfRange;
      dma_to_lds<16>(rs_ex, lds_addr(sc), off_add(lane * (int)kq, ks));
      dma_to_lds<16>(rs_ew, lds_addr(sc + 1024), off_add(lane * (int)kq, ks));
      dma_to_lds<16>(rs_ew, lds_addr(sc + 2048), off_add((64 + lane) * (int)kq, ks));
    }
  };

  // Fragment reads: row r = 16 t + (lane & 15) of the stage, chunks (2g, 2g+1)
  // (K 32g..32g+31), except for the scaled instruction on MX and MXFP4
  // operands, whose lane group g must hold 32-K block g: chunks (g, 4+g).
  const int swz = lds_swz(lane & 15);
  constexpr bool kPairedChunks = PATH == PATH_EXACT || (MODE != MODE_MX && !FP4);
  const int c0 = ((kPairedChunks ? 2 * g : g) ^ swz) << 4;
  const int c1 = ((kPairedChunks ? 2 * g + 1 : 4 + g) ^ swz) << 4;
  const int rlane = (lane & 15) * 128;
  bool hi[T];
#pragma unroll
  for (int t = 0; t < T; ++t) hi[t] = (n0 + 16 * t + (lane & 15)) / 128 > blo;

  v4f acc[MT][T];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[mt][t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  auto lds16 = [&](const uint8_t* b, int off) { return *reinterpret_cast<const u32x4*>(b + off); };

  auto compute = [&](int stage, int k) {
    const uint8_t* st = &lds[w][stage][0];
    const uint8_t* sc = st + St::kW + St::kX;
    float f_lo[MT][4], f_hi[MT][4];
    if constexpr (MODE == MODE_PROMOTE) {
      const float s_lo = reinterpret_cast<const float*>(sc + 256)[0];
      const float s_hi = reinterpret_cast<const float*>(sc + 256)[1];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const float4 sx4 = *reinterpret_cast<const float4*>(sc + (16 * mt + 4 * g) * 4);
        const float sx[4] = {sx4.x, sx4.y, sx4.z, sx4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f_lo[mt][r] = sx[r] * s_lo;
          f_hi[mt][r] = sx[r] * s_hi;
        }
      }
    }
    uint32_t ea[MT], eb[T];
    if constexpr (MODE == MODE_MX) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        ea[mt] = (reinterpret_cast<const uint32_t*>(sc)[16 * mt + (lane & 15)] >> (8 * g)) & 0xffu;
#pragma unroll
      for (int t = 0; t < T; ++t)
        eb[t] = (reinterpret_cast<const uint32_t*>(sc + 256)[16 * t + (lane & 15)] >> (8 * g)) & 0xffu;
    }
    if constexpr (MX4) {
      // Two FP4 instructions per step: half h takes chunk 4h + g of each row
      // (K 128h + 32g .. +31), which is MX block 4h + g, scaled by byte g of
      // the row's scale word h (MODE_MX4_PAIRS: word 2 (k & 1) + h of the
      // row's four).
      const uint32_t* sw32 = reinterpret_cast<const uint32_t*>(sc);
      auto words = [&](int xw, int row) {   // xw: 0 for X rows, 1 for W rows
        if constexpr (PAIRS) {
          return *reinterpret_cast<const uint2*>(sw32 + 256 * xw + 4 * row + 2 * (k & 1));
        } else {
          return uint2{sw32[128 * xw + row], sw32[64 + 192 * xw + row]};
        }
      };
      u32x4 al[MT], ah[MT];
      int ea0[MT], ea1[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = St::kW + 16 * mt * 128 + rlane;
        al[mt] = lds16(st, r + c0);
        ah[mt] = lds16(st, r + c1);
        const uint2 e = words(0, 16 * mt + (lane & 15));
        ea0[mt] = (int)((e.x >> (8 * g)) & 0xffu);
        ea1[mt] = (int)((e.y >> (8 * g)) & 0xffu);
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int r = 16 * t * 128 + rlane;
        const u32x4 bl = lds16(st, r + c0), bh = lds16(st, r + c1);
        const uint2 e = words(1, 16 * t + (lane & 15));
        const int eb0 = (int)((e.x >> (8 * g)) & 0xffu);
        const int eb1 = (int)((e.y >> (8 * g)) & 0xffu);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt][t] = mfma_fp4(al[mt], bl, acc[mt][t], ea0[mt], eb0);
          acc[mt][t] = mfma_fp4(ah[mt], bh, acc[mt][t], ea1[mt], eb1);
        }
      }
    } else if constexpr (MODE == MODE_NV4) {
      // NVFP4: the lane's chunks 2g and 2g+1 hold K 64g .. 64g+63 of the step,
      // NV blocks 4g .. 4g+3; chunk h is four fp16 operands of 8 codes, each
      // code times its E4M3 microscale (exact in fp16): words 0-1 of the chunk
      // take byte 2h of the row's scale word g, words 2-3 byte 2h+1.
      const uint32_t* sw32 = reinterpret_cast<const uint32_t*>(sc);
      auto frag = [&](int off, uint32_t mw, int h, v8h* x) {
        const u32x4 d = lds16(st, off + (h ? c1 : c0));
        v2h m0, m1;
        e4m3_pair_f16(mw, h, m0, m1);
        x[0] = cvt8_fp4_f16(d.x, m0);
        x[1] = cvt8_fp4_f16(d.y, m0);
        x[2] = cvt8_fp4_f16(d.z, m1);
        x[3] = cvt8_fp4_f16(d.w, m1);
      };
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v8h xa[MT][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          frag(St::kW + 16 * mt * 128 + rlane, sw32[4 * (16 * mt + (lane & 15)) + g], h, xa[mt]);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          v8h xb[4];
          frag(16 * t * 128 + rlane, sw32[256 + 4 * (16 * t + (lane & 15)) + g], h, xb);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) acc[mt][t] = mfma_f16(xa[mt][s4], xb[s4], acc[mt][t]);
        }
      }
    } else if constexpr (PATH == PATH_FAST) {
      v8i fa[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = St::kW + 16 * mt * 128 + rlane;
        fa[mt] = join(lds16(st, r + c0), lds16(st, r + c1));
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int r = 16 * t * 128 + rlane;
        const v8i fb = join(lds16(st, r + c0), lds16(st, r + c1));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if constexpr (MODE == MODE_PROMOTE) {
            const v4f pr = mfma_fp8<AF, BF>(fa[mt], fb, v4f{0.0f, 0.0f, 0.0f, 0.0f}, (int)kUnitScale, (int)kUnitScale);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[mt][t][q] = __builtin_fmaf(pr[q], hi[t] ? f_hi[mt][q] : f_lo[mt][q], acc[mt][t][q]);
          } else if constexpr (MODE == MODE_MX) {
            acc[mt][t] = mfma_fp8<AF, BF>(fa[mt], fb, acc[mt][t], (int)ea[mt], (int)eb[t]);
          } else {
            acc[mt][t] = mfma_fp8<AF, BF>(fa[mt], fb, acc[mt][t], (int)kUnitScale, (int)kUnitScale);
          }
        }
      }
    } else {
      // MX steps whose UE8M0 exponents leave the range in which folding 2^e
      // into an operand's bf16 conversion is exact and finite go block by
      // block: one 32-K block per instruction on unit-scale expansions (exact),
      // each block's fp32 sum added times 2^(eA + eB) with an exact ldexp.
      bool mx_wide = false;
      if constexpr (MODE == MODE_MX) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) mx_wide |= !mx_fold_exact<AF>(ea[mt]);
#pragma unroll
        for (int t = 0; t < T; ++t) mx_wide |= !mx_fold_exact<BF>(eb[t]);
        mx_wide = __builtin_amdgcn_ballot_w64(mx_wide) != 0;
      }
      if (MODE == MODE_MX && mx_wide) {
        const uint32_t* sw32 = reinterpret_cast<const uint32_t*>(sc);
#pragma unroll 1
        for (int b = 0; b < 4; ++b) {
          // lane group g: K 32b + 8g .. +7 of its row (logical chunk 2b + g/2)
          const int cb = (((2 * b + (g >> 1)) ^ swz) << 4) + 8 * (g & 1);
          v8bf xab[MT];
          int eam[MT][4];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const uint2 d = *reinterpret_cast<const uint2*>(st + St::kW + 16 * mt * 128 + rlane + cb);
            xab[mt] = cvt8<AF>(d.x, d.y, 1.0f);
            // X scale words of the tile's output rows 4g .. 4g+3
            const u32x4 wq = *reinterpret_cast<const u32x4*>(sw32 + 16 * mt + 4 * g);
            eam[mt][0] = (int)((wq.x >> (8 * b)) & 0xffu) - 127;
            eam[mt][1] = (int)((wq.y >> (8 * b)) & 0xffu) - 127;
            eam[mt][2] = (int)((wq.z >> (8 * b)) & 0xffu) - 127;
            eam[mt][3] = (int)((wq.w >> (8 * b)) & 0xffu) - 127;
          }
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const uint2 d = *reinterpret_cast<const uint2*>(st + 16 * t * 128 + rlane + cb);
            const v8bf xbb = cvt8<BF>(d.x, d.y, 1.0f);
            // the lane's own W row (its output column)
            const int ebt = (int)((sw32[64 + 16 * t + (lane & 15)] >> (8 * b)) & 0xffu) - 127;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const v4f pb = mfma_bf16(xab[mt], xbb, v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
              for (int q = 0; q < 4; ++q) acc[mt][t][q] += __builtin_amdgcn_ldexpf(pb[q], eam[mt][q] + ebt);
            }
            __builtin_amdgcn_sched_barrier(0);   // one column tile at a time (register pressure)
          }
        }
      } else {
      // X expanded once per step and reused for every column tile.
      v8bf xa[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const float fsa = (MODE == MODE_MX) ? e8m0_to_f32(ea[mt]) : 1.0f;
        const int r = St::kW + 16 * mt * 128 + rlane;
        const u32x4 d0 = lds16(st, r + c0), d1 = lds16(st, r + c1);
        xa[mt][0] = cvt8<AF>(d0.x, d0.y, fsa);
        xa[mt][1] = cvt8<AF>(d0.z, d0.w, fsa);
        xa[mt][2] = cvt8<AF>(d1.x, d1.y, fsa);
        xa[mt][3] = cvt8<AF>(d1.z, d1.w, fsa);
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float fsb = (MODE == MODE_MX) ? e8m0_to_f32(eb[t]) : 1.0f;
        const int r = 16 * t * 128 + rlane;
        const u32x4 d0 = lds16(st, r + c0), d1 = lds16(st, r + c1);
        v8bf xb[4];
        xb[0] = cvt8<BF>(d0.x, d0.y, fsb);
        xb[1] = cvt8<BF>(d0.z, d0.w, fsb);
        xb[2] = cvt8<BF>(d1.x, d1.y, fsb);
        xb[3] = cvt8<BF>(d1.z, d1.w, fsb);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if constexpr (MODE == MODE_PROMOTE) {
            v4f pp = mfma_bf16(xa[mt][0], xb[0], v4f{0.0f, 0.0f, 0.0f, 0.0f});
            pp = mfma_bf16(xa[mt][1], xb[1], pp);
            pp = mfma_bf16(xa[mt][2], xb[2], pp);
            pp = mfma_bf16(xa[mt][3], xb[3], pp);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[mt][t][q] = __builtin_fmaf(pp[q], hi[t] ? f_hi[mt][q] : f_lo[mt][q], acc[mt][t][q]);
          } else {
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) acc[mt][t] = mfma_bf16(xa[mt][s4], xb[s4], acc[mt][t]);
          }
        }
      }
      }
    }
  };

  // NS stages per wave (private: no workgroup barrier in the loop).  The
  // loads of steps k+1 .. k+NS-1 are in flight while step k is computed; the
  // explicit wait leaves exactly those loads outstanding.  Steps past the
  // wave's range load zeros and are not computed, so every iteration issues
  // the same number of loads.
  if (kb0 < kb1) {
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) issue(kb0 + j, j);
    int cs = 0;  // stage of step k
    for (int k = kb0; k < kb1; ++k) {
      issue(k + NS - 1, cs == 0 ? NS - 1 : cs - 1);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 1) * St::kLoads) : "memory");
      compute(cs, k);
      cs = cs + 1 == NS ? 0 : cs + 1;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the last (zero) loads have landed

  // Partial tiles of the S waves -> LDS (each wave's own stages) -> one sum
  // per output element.
  float* red = reinterpret_cast<float*>(&lds[w][0][0]);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < T; ++t)
      *reinterpret_cast<float4*>(&red[((mt * T + t) * 64 + lane) * 4]) =
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
      for (int s = 0; s < S; ++s) v += reinterpret_cast<const float*>(&lds[s][0][0])[(u * 64 + lane) * 4 + r];
      if (row >= M) continue;
      if constexpr (MODE == MODE_EPILOGUE) v = v * (sxa[p.a_per_row ? row : 0] * swb[p.b_per_row ? col : 0]);
      if constexpr (MODE == MODE_NV4) v = v * (p.ta[0] * p.tb[0]);
      store_out<ODT>(p.out, row * p.ldo + col, v);
    }
  }
}

// Literal launch bounds (a template-dependent bound leaves the host stubs
// undefined).
template <int AF, int BF, int MODE, int ODT, int PATH, int MT, int T>
__global__ __launch_bounds__(256) void k_gemm_skinny(GemmArgs p, int R) {
  gemm_skinny_body<AF, BF, MODE, ODT, PATH, MT, T, 4, 2>(p, R);  // 3 stages measured no faster
}

// ---- dispatch ----------------------------------------------------------------
// Up to 5 column tiles per workgroup (R <= 80 rows) for every M: one
// workgroup per CU up to N = 80 * CUs (the stages of M = 64 take 148 KB of
// LDS; fewer tiles per workgroup would need several workgroups per CU, each
// reading all of X, and measured slower).  The grid is c * CUs workgroups with
// the smallest c that keeps R within that bound.
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
  else if (mt <= 2) skinny_launch<AF, BF, MODE, ODT, PATH, 2, 5>(p, st);
  else skinny_launch<AF, BF, MODE, ODT, PATH, 4, 5>(p, st);
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

// FP4 operands (K % 256 == 0): MXFP4 on the FP4 matrix cores, NVFP4 on exact
// fp16 expansions.  NVFP4 stages four scale words per row and step, so with
// four X tiles (M > 32) a workgroup takes four column tiles to stay within the
// 160 KiB of LDS.
template <int ODT>
static void skinny_nv(const GemmArgs& p, hipStream_t st) {
  const int64_t mt = (p.M + 15) / 16;
  if (mt <= 1) skinny_launch<FMT_E4M3, FMT_E4M3, MODE_NV4, ODT, PATH_EXACT, 1, 5>(p, st);
  else if (mt <= 2) skinny_launch<FMT_E4M3, FMT_E4M3, MODE_NV4, ODT, PATH_EXACT, 2, 5>(p, st);
  else skinny_launch<FMT_E4M3, FMT_E4M3, MODE_NV4, ODT, PATH_EXACT, 4, 4>(p, st);
}

// MXFP4 with K % 512 == 0 and M <= 32 stages the scale bytes of step pairs
// row by row (MODE_MX4_PAIRS); with four X tiles that stage would not fit
// five column tiles in LDS, so M > 32 stages word by word.
template <int ODT>
static void skinny_mx4(const GemmArgs& p, hipStream_t st) {
  const int64_t mt = (p.M + 15) / 16;
  const bool pairs = p.K % 512 == 0;
  if (mt <= 1 && pairs) skinny_launch<FMT_E4M3, FMT_E4M3, MODE_MX4_PAIRS, ODT, PATH_FAST, 1, 5>(p, st);
  else if (mt <= 1) skinny_launch<FMT_E4M3, FMT_E4M3, MODE_MX4, ODT, PATH_FAST, 1, 5>(p, st);
  else if (mt <= 2 && pairs) skinny_launch<FMT_E4M3, FMT_E4M3, MODE_MX4_PAIRS, ODT, PATH_FAST, 2, 5>(p, st);
  else if (mt <= 2) skinny_launch<FMT_E4M3, FMT_E4M3, MODE_MX4, ODT, PATH_FAST, 2, 5>(p, st);
  else skinny_launch<FMT_E4M3, FMT_E4M3, MODE_MX4, ODT, PATH_FAST, 4, 5>(p, st);
}

hipError_t launch_gemm_skinny_fp4(const GemmArgs& p, int mode, int odt, hipStream_t st) {
  if (mode == MODE_NV4) {
    if (odt == DT_F32) skinny_nv<DT_F32>(p, st);
    else skinny_nv<DT_BF16>(p, st);
  } else if (odt == DT_F32) {
    skinny_mx4<DT_F32>(p, st);
  } else {
    skinny_mx4<DT_BF16>(p, st);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_skinny(const GemmArgs& p, int afmt, int bfmt, int mode, int odt, int path, hipStream_t st) {
  if (afmt == FMT_E4M3 && bfmt == FMT_E4M3) skinny_mode<FMT_E4M3, FMT_E4M3>(p, mode, odt, path, st);
  else if (afmt == FMT_E4M3) skinny_mode<FMT_E4M3, FMT_E5M2>(p, mode, odt, path, st);
  else if (bfmt == FMT_E4M3) skinny_mode<FMT_E5M2, FMT_E4M3>(p, mode, odt, path, st);
  else skinny_mode<FMT_E5M2, FMT_E5M2>(p, mode, odt, path, st);
  return hipGetLastError();
}

}  // namespace fp8blk
