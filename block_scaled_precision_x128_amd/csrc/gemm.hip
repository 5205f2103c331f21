// Block-scaled FP8 GEMM kernels for gfx950.
//
//   out[m, n] = sum_k decode(a[m,k]) sA(m,k) * decode(b[n,k]) sB(n,k)
//
// ("The FP8 Family": the MMA identity Out = s_X s_W (X_fp8 @ W_fp8^T) with an
// fp32 accumulator, and the DeepSeek-V3 callout's promotion to full fp32 every
// 128 K; "Illustrated GPU kernels, Part 8": the promotion paragraph and the
// OCP MX paragraph.)
//
// Two matrix-core paths compute the products:
//
//  PATH_EXACT (default): the FP8 codes stay FP8 in HBM and LDS and are
//    expanded in registers to bf16 (v_cvt_scalef32_pk_bf16_fp8, exact for
//    E4M3 and E5M2), then multiplied with v_mfma_f32_16x16x32_bf16, whose
//    products are exact and whose sums are fp32.  Lane l holds 32 consecutive
//    K bytes of row l%16 (K bytes 32*(l/16)..+31 of the 128-K step); the
//    step is four K=32 instructions, sub-step s taking bytes 8s..8s+7 of
//    every lane.  An MX block is then exactly one lane's 32 bytes, so its
//    power-of-two scale is folded into the bf16 conversion.
//
//  PATH_FAST: v_mfma_scale_f32_16x16x128_f8f6f4 on the codes (twice the peak
//    rate).  Its hardware K order is: lane group g = l/16 holds K 16g..16g+15
//    in bytes 0-15 and K 64+16g..64+16g+15 in bytes 16-31; the UE8M0 scale of
//    32-K block b comes from lane group b.  MX operands are loaded in exactly
//    that order (chunks g and 4+g of the row); otherwise lane group g loads
//    chunks 2g, 2g+1 (a permutation of K applied to both operands).  The instruction adds its products
//    eight at a time in a fixed-point window 14 bits below the largest of the
//    eight (smaller products are truncated) before the fp32 sum, so this path
//    does not meet the fp32-accumulation error bound on every input.
//
// In both, the 16x16 result tile is held as lane l: rows 4*(l/16)+r
// (r = 0..3), column l%16.
//
// Scale modes:
//   MODE_EPILOGUE  per-tensor / per-row scales: fp32 accumulation over all of
//                  K, one multiply by sA*sB at the end
//   MODE_PROMOTE   1x128 tiles x 128x128 blocks: each 128-K step gives a fresh
//                  partial product P that is added as acc += P * sA[m,kb]
//                  sB[n/128,kb] in fp32 on the vector ALU (the DeepSeek-V3
//                  promotion, once per 128-K step)
//   MODE_MX        32-element UE8M0 blocks: 2^(eA+eB) applied per 32-K block,
//                  folded into the bf16 operands (exact path) or given to the
//                  scaled MFMA (fast path)
//   MODE_MX4       MXFP4 (E2M1 codes, UE8M0 per 32): the FP4 form of the
//                  scaled MFMA, which sums each 32-element block exactly
//                  (E2M1 products need at most 13 bits) and adds the block
//                  sums in fp32, so it keeps the exact path's error bound
//   MODE_NV4       NVFP4 (E2M1 codes, E4M3 microscale per 16, fp32 tensor
//                  scales): codes times microscales expanded exactly to fp16
#include <type_traits>

#include "gemm_common.h"

namespace fp8blk {

// MODE_MX4_PAIRS (an even number of 256-K steps): a row's UE8M0 bytes of
// steps 2p and 2p+1 (16 bytes, 16-byte aligned since the row holds K/32
// bytes, a multiple of 16) are staged with one 16-byte load at step 2p into a
// two-slot ring, halving the scale loads.  Otherwise as MODE_MX4.

// ---------------------------------------------------------------------------
// Tiled kernel: a workgroup of 8 waves (2 along M x 4 along N) computes a
// 256x256 output tile (wave tiles 128x64; 256x192 and 128x256 variants
// below), in 128-K steps.  Both operand tiles are FP8 in LDS, in two or three
// stages; global data goes to LDS with buffer_load ... lds (no register
// staging), through descriptors that cover only the tile's valid rows, so
// rows past M or N arrive as zeros.  One barrier per K step, after which the
// stage of step k-1 is free: the loads of step k+NS-1 go there, issued a few
// at a time from the first half of step k's multiply loop, and land while
// later steps compute.
//
// LDS tile layout: 128-byte rows of eight 16-byte chunks; chunk c of row r is
// stored at chunk c ^ swz(r), swz(r) = (r & 7) ^ ((r >> 3) & 1).  A fragment
// read has each 16-lane group fetch one chunk from each of 16 consecutive
// rows; with this swizzle those reads are free of LDS bank conflicts on
// gfx950 (measured with SQ_LDS_BANK_CONFLICT; the plain r & 7 and (r >> 1) & 7
// swizzles both stall 4 cycles per ds_read_b128).
// ---------------------------------------------------------------------------
constexpr int TBK = 128;

// Workgroup id -> output tile.  Consecutive ids are dispatched round-robin
// over the 8 XCDs; each XCD is given a contiguous run of logical tiles, and
// logical tiles walk groups of 8 tile-rows column by column, so the tiles
// that share rows of A or B run on the same XCD and share its L2.
__device__ __forceinline__ void tile_coords(int64_t bid, int64_t ntm, int64_t ntn, int64_t& tm, int64_t& tn) {
  const int64_t nb = ntm * ntn;
  const int64_t xcd = bid & 7, idx = bid >> 3;
  const int64_t q = nb >> 3, r = nb & 7;
  const int64_t logical = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
  constexpr int64_t GM = 8;
  const int64_t group_size = GM * ntn;
  const int64_t g = logical / group_size;
  const int64_t first_m = g * GM;
  const int64_t gm = (ntm - first_m) < GM ? (ntm - first_m) : GM;
  const int64_t in_g = logical - g * group_size;
  tm = first_m + in_g % gm;
  tn = in_g / gm;
}



template <int AF, int BF, int MODE, int ODT, int PATH, int WMW, int WNW, int MI, int NJ, int NS>
__device__ __forceinline__ void gemm_tiled_body(const GemmArgs& p) {
  constexpr int WR = 16 * MI, WC = 16 * NJ;            // wave tile: MI x NJ 16x16 output tiles
  constexpr int TBM = WR * WMW, TBN = WC * WNW;        // workgroup tile
  constexpr int NW = WMW * WNW;                        // waves
  constexpr int LPW = (TBM + TBN) / 8 / NW;            // 1-KiB loads per wave per K step
  static_assert((TBM + TBN) % (8 * NW) == 0, "rows must split evenly over the waves");
  // FP4 operands: two codes per byte, so a K step of 128 bytes per row holds 256 K.
  constexpr bool PAIRS = MODE == MODE_MX4_PAIRS;
  constexpr bool MX4 = MODE == MODE_MX4 || PAIRS;
  constexpr bool FP4 = MX4 || MODE == MODE_NV4;
  // MXFP4 runs on the FP4 matrix cores (PATH_FAST); NVFP4's E4M3 microscales
  // are not powers of two, so its codes are expanded (PATH_EXACT).
  static_assert(MODE != MODE_NV4 || PATH == PATH_EXACT, "NVFP4 operands take the exact path");
  static_assert(!MX4 || PATH == PATH_FAST, "MXFP4 operands take the FP4 matrix cores");
  // Scale words staged per row and step: FP8 MX 4 bytes (128 K / 32), MXFP4 8
  // bytes (256 K / 32), NVFP4 16 bytes (256 K / 16).
  // NVFP4 stages a row's 16 bytes with one 16-byte load (s_e then holds 4
  // consecutive words per row), MODE_MX4_PAIRS two steps' 8 bytes the same
  // way on even steps only; MX and MODE_MX4 stage word by word.
  constexpr int SW = MODE == MODE_MX4 ? 2 : (MODE == MODE_NV4 || PAIRS ? 4 : 1);
  constexpr int SCALE_CHUNKS = MODE == MODE_PROMOTE ? TBM / 64 + 1
                               : (MODE == MODE_NV4 || PAIRS ? (TBM + TBN) / 64
                                                            : (MODE == MODE_MX || FP4 ? SW * (TBM + TBN) / 64 : 0));
  constexpr int SC = (SCALE_CHUNKS + NW - 1) / NW;     // scale loads per wave per (even) step
  constexpr int LOADS = LPW + SC;                      // loads per wave per step (MODE_MX4_PAIRS: even steps)
  constexpr int ES = PAIRS ? 2 : NS;                   // scale stages
  constexpr bool MX_WORDS = MODE == MODE_MX && PATH == PATH_EXACT;   // exact MX: scale words read per step
  static_assert((NS - 1) * LOADS <= 63, "loads in flight must fit the vmcnt counter");
  static_assert(TBM % 64 == 0 && (TBM + TBN) % 64 == 0, "scale loads move 64 rows at a time");
  // NS LDS stages; the loads of the next NS-1 K steps are in flight while one is computed.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS][(TBM + TBN) * TBK];
  __shared__ __attribute__((aligned(16))) float s_x[NS][TBM];                    // MODE_PROMOTE: sA[m, kb]
  __shared__ __attribute__((aligned(16))) uint32_t s_e[ES][SW][TBM + TBN];       // MX / FP4: scale words per row
  __shared__ __attribute__((aligned(16))) float s_w[NS][64];                     // MODE_PROMOTE: sB[n/128, kb]
  __shared__ __attribute__((aligned(16))) uint32_t s_spare[64];                  // target of filler loads

  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t ntm = (M + TBM - 1) / TBM, ntn = (N + TBN - 1) / TBN;
  int64_t tm, tn;
  tile_coords(blockIdx.x, ntm, ntn, tm, tn);
  const int64_t m0 = tm * TBM, n0 = tn * TBN;
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w / WNW, wn = w % WNW;  // wave tile: rows wm*WR.., cols wn*WC..
  const int64_t KB = FP4 ? K / 2 : K;                  // bytes per operand row
  const int nkb = (int)(KB / 128);
  const int64_t rows_a = (M - m0) < TBM ? (M - m0) : TBM;
  const int64_t rows_b = (N - n0) < TBN ? (N - n0) : TBN;

  // The row-block loads of step kb + NS - 1 are issued from inside step kb's
  // multiply loop, a few at a time, rather than all at once after the
  // barrier.  A burst of load instructions there stalls the waves that issue
  // it while both waves of every SIMD are converting their B operands, and the
  // matrix cores idle; inside the loop the loads overlap the other wave's
  // multiplies.  Measured against the burst (A/B on one box, outputs
  // bit-identical): exact promotion 256x256 tiles at 4096x7168x7168 6% faster
  // (the 256x192 tiles, more VALU-bound, gained nothing), the FP8 native loop
  // 2% at 4096x7168x7168 and 8192^3, the exact MX loop 1.4% at 8192^3, the
  // MXFP4 loop 3%, and with three stages (128x256 tiles) the native loop 7.5%
  // at 2048x4096x4096 (exact 0-2%); then, issued over the first half of the
  // loop (issue_part below), the NVFP4 loop 1.6%.

  // The TBM A rows and TBN B rows of a K step form one list of LDS rows,
  // 8 rows (1 KiB) per load instruction; wave w issues instructions
  // [w*LPW, w*LPW + LPW).  Lane q lands in row 8u + q/8, stored chunk q%8,
  // which holds logical chunk (q%8) ^ lds_swz(row).
  // Row 8x + q/8 has lds_swz = (q/8) ^ (x & 1), so a lane's offset inside its
  // 8-row block is one of two per-lane values.  Descriptors cover only the
  // tile's valid rows (rows past M or N read zeros).  The block is selected by
  // a wave-uniform offset added to the lane's offset inside the load's
  // assembly, in one descriptor per operand (a descriptor per block, kept live
  // through the multiply loop, costs scalar registers; offsets precomputed by
  // the compiler cost a vector register per load).  Offsets stay below
  // 384 * K <= 1.5 * 2^30 bytes, and below 2^32 with the filler loads'
  // kOutOfRange added (unsigned 32-bit offsets).
  const int q8 = lane >> 3;
  const int goff_even = q8 * (int)KB + (((lane & 7) ^ q8) << 4);
  const int goff_odd = q8 * (int)KB + (((lane & 7) ^ q8 ^ 1) << 4);
  const uint8_t* a_base = p.a + m0 * KB;
  const uint8_t* b_base = p.b + n0 * KB;
  const __amdgpu_buffer_rsrc_t rs_a = uniform_rsrc(a_base, rows_a * KB), rs_b = uniform_rsrc(b_base, rows_b * KB);

  // Scale descriptors (same row ranges) and per-lane offsets of the staged scales.
  const int64_t kq = MODE == MODE_NV4 ? K / 16 : K / 32;   // scale bytes per row
  __amdgpu_buffer_rsrc_t rssa = rs_a, rssb = rs_b;
  if constexpr (MODE == MODE_PROMOTE)
    rssa = uniform_rsrc(reinterpret_cast<const float*>(p.sa) + m0 * nkb, rows_a * nkb * 4);
  if constexpr (MODE == MODE_MX || FP4) {
    rssa = uniform_rsrc(reinterpret_cast<const uint8_t*>(p.sa) + m0 * kq, rows_a * kq);
    rssb = uniform_rsrc(reinterpret_cast<const uint8_t*>(p.sb) + n0 * kq, rows_b * kq);
  }
  const float* swb = reinterpret_cast<const float*>(p.sb);
  const float* sxa = reinterpret_cast<const float*>(p.sa);
  // W block scales: blocks n0/128 .. (n0 + rows_b - 1)/128 (MODE_PROMOTE)
  const int64_t wblk0 = n0 / 128, wblks = (n0 + rows_b + 127) / 128 - wblk0;
  const __amdgpu_buffer_rsrc_t rssw = uniform_rsrc(swb + wblk0 * nkb, MODE == MODE_PROMOTE ? wblks * nkb * 4 : 0);

  // This wave's row-block loads u0 .. u1-1 of step kb into stage buf (kb < 0:
  // loads past every descriptor, which read nothing and fill the stage with
  // zeros; a stage no step reads).
  // The LDS address of stage 0 in a scalar register: each load's M0 is then
  // formed by scalar adds (from a vector register it took a vector add and a
  // readfirstlane per load, 16 vector instructions per step; 1.3% faster at
  // 4096x7168x7168 on both paths, A/B on one box, outputs bit-identical).
  const uint32_t smem_s = __builtin_amdgcn_readfirstlane(lds_addr(&smem[0][0]));
  auto issue_rows = [&](int kb, int buf, int u0, int u1) {
    const int kk = kb < 0 ? kOutOfRange : kb * 128;
#pragma unroll
    for (int u = u0; u < u1; ++u) {
      const int x = w * LPW + u;       // 8-row block of the A+B list (wave-uniform)
      const bool is_a = 8 * x < TBM;   // wave-uniform: scalar selects, no branch
      const int xl = is_a ? x : x - TBM / 8;
      const int goff = (x & 1) ? goff_odd : goff_even;
      dma16_to_lds_add(is_a ? rs_a : rs_b, smem_s + (uint32_t)(buf * ((TBM + TBN) * TBK) + 8 * x * 128), goff,
                       __builtin_amdgcn_readfirstlane(off_add(xl * 8 * (int)KB, kk)));
    }
  };
  // Row blocks u0 .. u1-1 of step kb + NS - 1, into the stage that step kb's
  // barrier freed (the stage step kb - 1 read); filler loads past the last step.
  auto issue_next = [&](int kb, int buf, int u0, int u1) {
    const int nxt = kb + NS - 1;
    issue_rows(nxt < nkb ? nxt : -1, buf == 0 ? NS - 1 : buf - 1, u0, u1);
  };
  // Inside the multiply loop, tile t of the first P tiles issues its share
  // (LPW / P) of those row blocks, so they are all in flight by the middle of
  // the step.  Spread over the whole loop (odd tiles), the last ones went out
  // too late to land before the next step's wait: issuing them over the first
  // half measured 4% faster on the exact path (4096x7168x7168 and 8192^3) and
  // 6% on the native one (A/B on one box, outputs bit-identical); over the
  // first quarter, or all at the first tile, was slower than the first half.
  auto issue_part = [&](int kb, int buf, int t, int P) {
    if (t >= 0 && t < P) issue_next(kb, buf, t * LPW / P, (t + 1) * LPW / P);
  };
  auto issue_loads = [&](int kb, int buf, bool rows) {
    if (rows) issue_rows(kb, buf, 0, LPW);
    // Scales, 64 rows per 4-byte load, spread so that every wave issues
    // exactly SC of them per step (a wave with no chunk left loads zeros into
    // a spare slot): every wave then issues the same number of loads per
    // step, which the multi-stage wait below counts on.
    if constexpr (MODE == MODE_PROMOTE) {
#pragma unroll
      for (int t2 = 0; t2 < SC; ++t2) {
        const int c = w + NW * t2;   // chunks 0 .. TBM/64-1: sA rows; chunk TBM/64: the W block scales
        if (c < TBM / 64)
          dma_to_lds<4>(rssa, lds_addr(&s_x[buf][64 * c]), ((64 * c + lane) * nkb + kb) * 4);
        else if (c == TBM / 64)
          dma_to_lds<4>(rssw, lds_addr(&s_w[buf][0]), (lane * nkb + kb) * 4);
        else
          dma_to_lds<4>(rssw, lds_addr(&s_spare[0]), kOutOfRange);
      }
    }
    if constexpr (MODE == MODE_NV4 || PAIRS) {
      // one 16-byte load per 64 rows: row R's words at s_e[slot] + 4 R
      // (MODE_MX4_PAIRS: steps kb, kb+1 into slot kb/2 % 2, at even kb only)
      constexpr int RC = (TBM + TBN) / 64;
      if (PAIRS && (kb & 1)) return;
      uint32_t* se = &s_e[PAIRS ? (kb >> 1) & 1 : buf][0][0];
#pragma unroll
      for (int t2 = 0; t2 < SC; ++t2) {
        const int c = w + NW * t2;
        if (c >= RC)
          dma_to_lds<4>(rssb, lds_addr(&s_spare[0]), kOutOfRange);
        else if (c < TBM / 64)
          dma_to_lds<16>(rssa, lds_addr(se + 4 * 64 * c), (int)((64 * c + lane) * kq + kb * (PAIRS ? 8 : 16)));
        else
          dma_to_lds<16>(rssb, lds_addr(se + 4 * 64 * c),
                         (int)((64 * c - TBM + lane) * kq + kb * (PAIRS ? 8 : 16)));
      }
    } else if constexpr (MODE == MODE_MX || FP4) {
      constexpr int RC = (TBM + TBN) / 64;   // row chunks; word wd of every row chunk is a chunk of its own
#pragma unroll
      for (int t2 = 0; t2 < SC; ++t2) {
        const int c = w + NW * t2;   // chunks of 64 rows: A rows first, then B rows, word by word
        const int wd = c / RC, rc = c - wd * RC;
        if (c >= SW * RC)
          dma_to_lds<4>(rssb, lds_addr(&s_spare[0]), kOutOfRange);
        else if (rc < TBM / 64)
          dma_to_lds<4>(rssa, lds_addr(&s_e[buf][wd][64 * rc]),
                        (int)((64 * rc + lane) * kq + kb * 4 * SW + 4 * wd));
        else
          dma_to_lds<4>(rssb, lds_addr(&s_e[buf][wd][64 * rc]),
                        (int)((64 * rc - TBM + lane) * kq + kb * 4 * SW + 4 * wd));
      }
    }
  };

  // Fragment reads: two 16-byte chunks of row r (r & 15 == lane & 15).
  // Chunks 2g, 2g+1 (K 32g..32g+31 of the step), except where the scaled
  // FP8/FP4 instruction pairs each 32-K block with one lane group's scale byte
  // (MX and MXFP4: chunks g, 4+g).  Outside MX the FP8 instruction's K order
  // is free (one instruction spans the whole 128-K step) and the paired chunks
  // measured 2-7% faster than (g, 4+g) at 4096x7168x7168 and 2048x4096x4096.
  const int g = lane >> 4, sw_ = lds_swz(lane & 15);
  constexpr bool kPairedChunks = PATH == PATH_EXACT || (MODE != MODE_MX && !FP4);
  const int c0 = ((kPairedChunks ? 2 * g : g) ^ sw_) << 4;
  const int c1 = ((kPairedChunks ? 2 * g + 1 : 4 + g) ^ sw_) << 4;
  const int a_row0 = wm * WR + (lane & 15);       // + 16 i
  const int b_row0 = wn * WC + (lane & 15);        // + 16 j
  // column block of this wave's columns (for 128x128 weight blocks); a wave
  // whose columns all lie past N (ragged last tile) reads the last block
  const int64_t nblk_raw = (n0 + wn * WC) / 128, nblk_max = (N + 127) / 128 - 1;
  const int64_t nblk = nblk_raw < nblk_max ? nblk_raw : nblk_max;
  // When a wave's columns can straddle a 128-column block (WC does not divide
  // 128), each lane takes the W block scale of its own column, per N tile.
  constexpr bool kWaveWScale = (128 % WC) == 0;
  // Exact promotion with such waves: the products are formed transposed (W
  // rows as the instruction's first operand), so a lane holds one output row
  // and four consecutive columns of each N tile; a 16-column tile never
  // straddles a 128-column block, so the scale of a lane's N tile is one
  // product sA * sB instead of four (256x192 tiles at 4096x7168x7168: one
  // multiply per MFMA instruction fewer, measured with SQ_INSTS_VALU_MUL_F32).
  constexpr bool kTransposed = !kWaveWScale && PATH == PATH_EXACT && MODE == MODE_PROMOTE;
  // Exact promotion on wave tiles wider than tall: A held for the step, B streamed
  // (the only layout that takes the transposed products).
  constexpr bool kStreamB = kTransposed && NJ > MI;
  static_assert(!kTransposed || kStreamB, "transposed products are formed by the streamed-B loop only");
  int jblk[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int64_t b = (n0 + wn * WC + 16 * j + (lane & 15)) / 128;
    jblk[j] = (int)((b < nblk_max ? b : nblk_max) - (n0 / 128));
  }

  v4f acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < nkb) issue_loads(j, j, true);


  // Wait for step kb's loads (those of later steps stay in flight: every wave
  // issues LOADS per step, and loads complete in issue order), publish the
  // stage to every wave, then reuse the stage read in the previous step for
  // step kb + NS - 1.
  auto sync_step = [&](int kb, int buf) {
    if constexpr (NS == 3) {
      // (MODE_MX4_PAIRS: odd steps issue no scale loads)
      if (kb + 1 < nkb) {
        if (PAIRS && ((kb + 1) & 1)) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPW) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS) : "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
    } else {
      static_assert(NS == 2, "two or three stages");
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    if (kb + NS - 1 < nkb) issue_loads(kb + NS - 1, buf == 0 ? NS - 1 : buf - 1, false);
  };

  int buf = 0;   // stage of step kb
  int kb = 0;
  bool mx_wide = false;   // exact MX: a step whose exponents cannot be folded (below)
  for (; kb < nkb; ++kb) {
    sync_step(kb, buf);
    if constexpr (MX_WORDS) {
      // Folding 2^e into an operand's bf16 expansion is exact and finite only
      // for e in a range (mx_fold_exact); the first step with an exponent
      // outside it (for any row of the wave) hands this and every later step
      // to the block-by-block loop below.
      bool w = false;
#pragma unroll
      for (int i = 0; i < MI; ++i) w |= !mx_fold_exact<AF>((s_e[buf][0][a_row0 + 16 * i] >> (8 * g)) & 0xffu);
#pragma unroll
      for (int j = 0; j < NJ; ++j) w |= !mx_fold_exact<BF>((s_e[buf][0][TBM + b_row0 + 16 * j] >> (8 * g)) & 0xffu);
      if (__builtin_amdgcn_ballot_w64(w) != 0) {
        mx_wide = true;
        break;
      }
    }

    const uint8_t* sa_ = &smem[buf][0];
    const uint8_t* sb_ = &smem[buf][TBM * TBK];
    auto lds16 = [&](const uint8_t* base, int off) { return *reinterpret_cast<const u32x4*>(base + off); };

    float swv = 1.0f, swj[NJ];
    if constexpr (MODE == MODE_PROMOTE) {
      if constexpr (kWaveWScale) {
        swv = s_w[buf][nblk - wblk0];
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) swj[j] = s_w[buf][jblk[j]];
      }
    }

    if constexpr (MX4) {
      // MXFP4 on the FP4 matrix cores: a 256-K step is two 128-K halves, one
      // instruction each.  In half h, lane group g holds chunk 4h + g of its
      // row (K 128h + 32g .. +31, element 2i in the low nibble of byte i),
      // which is exactly MX block 4h + g; its UE8M0 byte is byte g of staged
      // scale word h.  The instruction scales each block's products by
      // 2^(eA + eB) and sums every 32-element block exactly (E2M1 products
      // span at most 13 bits), then adds the four block sums in fp32.
      // Scale words (h = 0, 1) of row R: s_e[buf][h][R], or with
      // MODE_MX4_PAIRS words 2 (kb & 1) + h of row R's four in its slot.
      const uint32_t* sp = &s_e[(kb >> 1) & 1][0][0] + 2 * (kb & 1);
      auto scale_words = [&](int row) {
        if constexpr (PAIRS) {
          const uint2 v = *reinterpret_cast<const uint2*>(sp + 4 * row);
          return v;
        } else {
          return uint2{s_e[buf][0][row], s_e[buf][1][row]};
        }
      };
      u32x4 bl[NJ], bh[NJ];
      int eb0[NJ], eb1[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int r = b_row0 + 16 * j;
        bl[j] = lds16(sb_, r * 128 + c0);
        bh[j] = lds16(sb_, r * 128 + c1);
        const uint2 e = scale_words(TBM + r);
        eb0[j] = (int)((e.x >> (8 * g)) & 0xffu);
        eb1[j] = (int)((e.y >> (8 * g)) & 0xffu);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        issue_part(kb, buf, i, MI / 2);
        const int r = a_row0 + 16 * i;
        const u32x4 al = lds16(sa_, r * 128 + c0), ah = lds16(sa_, r * 128 + c1);
        const uint2 e = scale_words(r);
        const int ea0 = (int)((e.x >> (8 * g)) & 0xffu);
        const int ea1 = (int)((e.y >> (8 * g)) & 0xffu);
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_fp4(al, bl[j], acc[i][j], ea0, eb0[j]);
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_fp4(ah, bh[j], acc[i][j], ea1, eb1[j]);
      }
    } else if constexpr (PATH == PATH_FAST) {
      v8i fb[NJ];
      int eb[NJ] = {};
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int r = b_row0 + 16 * j;
        fb[j] = join(lds16(sb_, r * 128 + c0), lds16(sb_, r * 128 + c1));
        if constexpr (MODE == MODE_MX) eb[j] = (int)((s_e[buf][0][TBM + r] >> (8 * g)) & 0xffu);
      }
      // Outside promotion the next A fragment is read one tile ahead (MX: 2.6%
      // faster at 8192^3; with promotion it measured 2.7% slower at
      // 4096x7168x7168).
      constexpr bool kPrefetchA = MODE != MODE_PROMOTE;
      constexpr int kIssueFrom = MODE == MODE_PROMOTE ? 1 : 0;
      v8i fa_next = {};
      if constexpr (kPrefetchA) fa_next = join(lds16(sa_, a_row0 * 128 + c0), lds16(sa_, a_row0 * 128 + c1));
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        // with promotion the loads go out from the second tile on: 2-3% faster
        // at 4096x7168x7168 (two A/B runs on one box); the MX loop lost 2%
        // that way
        if (i >= kIssueFrom) issue_part(kb, buf, i - kIssueFrom, MI / 2);
        const int r = a_row0 + 16 * i;
        v8i fa;
        if constexpr (kPrefetchA) {
          fa = fa_next;
          if (i + 1 < MI) fa_next = join(lds16(sa_, (r + 16) * 128 + c0), lds16(sa_, (r + 16) * 128 + c1));
        } else {
          fa = join(lds16(sa_, r * 128 + c0), lds16(sa_, r * 128 + c1));
        }
        if constexpr (MODE == MODE_PROMOTE) {
          const float4 sx4 = *reinterpret_cast<const float4*>(&s_x[buf][wm * WR + 16 * i + 4 * g]);
          const v4f sc = {sx4.x * swv, sx4.y * swv, sx4.z * swv, sx4.w * swv};  // swv = 1 when per lane
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const v4f pr = mfma_fp8<AF, BF>(fa, fb[j], v4f{0.0f, 0.0f, 0.0f, 0.0f}, (int)kUnitScale, (int)kUnitScale);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][j][q] = __builtin_fmaf(pr[q], kWaveWScale ? sc[q] : sc[q] * swj[j], acc[i][j][q]);
          }
        } else if constexpr (MODE == MODE_MX) {
          const int ea = (int)((s_e[buf][0][r] >> (8 * g)) & 0xffu);
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_fp8<AF, BF>(fa, fb[j], acc[i][j], ea, eb[j]);
        } else {
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = mfma_fp8<AF, BF>(fa, fb[j], acc[i][j], (int)kUnitScale, (int)kUnitScale);
        }
      }
    } else if constexpr (MODE == MODE_NV4) {
      // NVFP4 exact path: the lane's two 16-byte chunks (2g, 2g+1) hold K
      // 64g..64g+63 of this 256-K step; each chunk is 32 codes, four matrix
      // operands of 8 (byte i of a word holds codes 2i, 2i+1 in its low and
      // high nibble).  Every code times its E4M3 microscale is exact in fp16,
      // applied by a packed fp16 multiply (the scaled converts keep only a
      // scale's exponent); words 0-1 and 2-3 of a chunk are blocks 4g+2h and
      // 4g+2h+1, bytes 2h and 2h+1 of staged word g.
      using Op = v8h;
      auto frag = [&](const uint8_t* base, int row, int R, int h, Op* x) {
        const u32x4 d = lds16(base, row * 128 + (h ? c1 : c0));
        const uint32_t mw = (&s_e[buf][0][0])[4 * R + g];
        v2h m0, m1;
        e4m3_pair_f16(mw, h, m0, m1);
        x[0] = cvt8_fp4_f16(d.x, m0);
        x[1] = cvt8_fp4_f16(d.y, m0);
        x[2] = cvt8_fp4_f16(d.z, m1);
        x[3] = cvt8_fp4_f16(d.w, m1);
      };
      auto mma = [](const Op& a, const Op& b, const v4f& c) { return mfma_f16(a, b, c); };
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        Op xb[NJ][4];
#pragma unroll
        for (int j = 0; j < NJ; ++j) frag(sb_, b_row0 + 16 * j, TBM + b_row0 + 16 * j, h, xb[j]);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          if (h == 0) issue_part(kb, buf, i, MI / 2);
          Op xa[4];
          frag(sa_, a_row0 + 16 * i, a_row0 + 16 * i, h, xa);
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[i][j] = mma(xa[s], xb[j][s], acc[i][j]);
        }
      }
    } else if constexpr (kStreamB) {
      // Exact promotion with A held for the step (wave tiles wider than they
      // are tall): the MI A tiles are converted once after the barrier, then
      // N tile j+1 is read and converted, and tile j-1's partials promoted,
      // while tile j multiplies (the deferred promotion measured 1.8% faster).  Products
      // transposed (kTransposed): lane l holds output row 16 i + l%16 and
      // columns 16 j + 4 g + q, so one sA * sB per (i, j).
      v8bf xa[MI][4];
      float sxl[MI];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = a_row0 + 16 * i;
        const u32x4 d0 = lds16(sa_, r * 128 + c0), d1 = lds16(sa_, r * 128 + c1);
        xa[i][0] = cvt8<AF>(d0.x, d0.y, 1.0f);
        xa[i][1] = cvt8<AF>(d0.z, d0.w, 1.0f);
        xa[i][2] = cvt8<AF>(d1.x, d1.y, 1.0f);
        xa[i][3] = cvt8<AF>(d1.z, d1.w, 1.0f);
        sxl[i] = s_x[buf][wm * WR + 16 * i + (lane & 15)];
      }
      u32x4 n0 = lds16(sb_, b_row0 * 128 + c0), n1 = lds16(sb_, b_row0 * 128 + c1);
      v8bf xbv[4];
      v4f ppd[MI];   // the previous N tile's partials, promoted under this tile's MFMAs
      xbv[0] = cvt8<BF>(n0.x, n0.y, 1.0f);
      xbv[1] = cvt8<BF>(n0.z, n0.w, 1.0f);
      xbv[2] = cvt8<BF>(n1.x, n1.y, 1.0f);
      xbv[3] = cvt8<BF>(n1.z, n1.w, 1.0f);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        // the next step's row blocks over the first half of the N tiles
        // (filler loads on the last step: no branch in the unrolled loop)
        issue_part(kb, buf, j, NJ / 2);
        if (j + 1 < NJ) {
          const int r = b_row0 + 16 * (j + 1);
          n0 = lds16(sb_, r * 128 + c0);
          n1 = lds16(sb_, r * 128 + c1);
        }
        __builtin_amdgcn_s_setprio(1);
        v4f pp[MI];
#pragma unroll
        for (int i = 0; i < MI; ++i) pp[i] = mfma_bf16(xbv[0], xa[i][0], v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
        for (int s = 1; s < 4; ++s)
#pragma unroll
          for (int i = 0; i < MI; ++i) pp[i] = mfma_bf16(xbv[s], xa[i][s], pp[i]);
        __builtin_amdgcn_s_setprio(0);
        if (j > 0) {
#pragma unroll
          for (int i = 0; i < MI; ++i) {
            const float sc = sxl[i] * swj[j - 1];
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][j - 1][q] = __builtin_fmaf(ppd[i][q], sc, acc[i][j - 1][q]);
          }
        }
#pragma unroll
        for (int i = 0; i < MI; ++i) ppd[i] = pp[i];
        if (j + 1 < NJ) {
          xbv[0] = cvt8<BF>(n0.x, n0.y, 1.0f);
          xbv[1] = cvt8<BF>(n0.z, n0.w, 1.0f);
          xbv[2] = cvt8<BF>(n1.x, n1.y, 1.0f);
          xbv[3] = cvt8<BF>(n1.z, n1.w, 1.0f);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int z = 0; z < 4 * MI; ++z) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const float sc = sxl[i] * swj[NJ - 1];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][NJ - 1][q] = __builtin_fmaf(ppd[i][q], sc, acc[i][NJ - 1][q]);
      }
    } else {
      // Exact path: four K=32 sub-steps on bf16 operands (MX scales folded in).
      v8bf xb[NJ][4];
      u32x4 bd[NJ][2];   // MODE_PROMOTE: B's codes, converted among A tile 0's multiplies (below)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int r = b_row0 + 16 * j;
        const u32x4 d0 = lds16(sb_, r * 128 + c0), d1 = lds16(sb_, r * 128 + c1);
        if constexpr (MODE == MODE_PROMOTE) {
          bd[j][0] = d0;
          bd[j][1] = d1;
        } else {
          const float fsb = (MODE == MODE_MX) ? e8m0_to_f32((s_e[buf][0][TBM + r] >> (8 * g)) & 0xffu) : 1.0f;
          xb[j][0] = cvt8<BF>(d0.x, d0.y, fsb);
          xb[j][1] = cvt8<BF>(d0.z, d0.w, fsb);
          xb[j][2] = cvt8<BF>(d1.x, d1.y, fsb);
          xb[j][3] = cvt8<BF>(d1.z, d1.w, fsb);
        }
      }
      if constexpr (MODE == MODE_PROMOTE) {
        // Software-pipelined order: A tile i+1 is read and converted while
        // tile i multiplies; each N tile's 128-K partial P is a chain of four
        // MFMAs, and the four chains of a tile row are interleaved before P
        // is promoted into the fp32 accumulator.
        u32x4 n0 = lds16(sa_, a_row0 * 128 + c0), n1 = lds16(sa_, a_row0 * 128 + c1);
        v8bf xa[4];
        xa[0] = cvt8<AF>(n0.x, n0.y, 1.0f);
        xa[1] = cvt8<AF>(n0.z, n0.w, 1.0f);
        xa[2] = cvt8<AF>(n1.x, n1.y, 1.0f);
        xa[3] = cvt8<AF>(n1.z, n1.w, 1.0f);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          // the next step's row blocks over the first half of the A tiles
          // (the last step issues filler loads: no branch inside the
          // unrolled loop, which measured to cost register spills)
          issue_part(kb, buf, i, MI / 2);
          if (i + 1 < MI) {
            const int r = a_row0 + 16 * (i + 1);
            n0 = lds16(sa_, r * 128 + c0);
            n1 = lds16(sa_, r * 128 + c1);
          }
          // scales of this A tile's rows (lane rows 16 i + 4 g + q), read before the multiplies
          const float4 sx4 = *reinterpret_cast<const float4*>(&s_x[buf][wm * WR + 16 * i + 4 * g]);
          const v4f sc = {sx4.x * swv, sx4.y * swv, sx4.z * swv, sx4.w * swv};  // swv = 1 when per lane
          // Four independent chains (one per N tile), interleaved so that
          // no MFMA waits on the previous one; the wave's priority is raised
          // while it issues them so that a co-resident wave's VALU work fills
          // the gaps instead of delaying the matrix cores.
          __builtin_amdgcn_s_setprio(1);
          v4f pp[NJ];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            // A tile 0 converts B's chunk s of every N tile just before the
            // multiplies that use it, four conversions before each MFMA, so
            // the matrix cores start 20 conversions into the step instead of
            // 80 (both waves of a SIMD leave the barrier together and would
            // otherwise convert at once): 2% faster at 4096x7168x7168 (A/B
            // on one box, outputs bit-identical); A tile 0 converted the
            // same way measured no better.
            if (i == 0) {
#pragma unroll
              for (int j = 0; j < NJ; ++j) {
                const u32x4 d = bd[j][s >> 1];
                xb[j][s] = (s & 1) ? cvt8<BF>(d.z, d.w, 1.0f) : cvt8<BF>(d.x, d.y, 1.0f);
              }
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j)
              pp[j] = mfma_bf16(xa[s], xb[j][s], s == 0 ? v4f{0.0f, 0.0f, 0.0f, 0.0f} : pp[j]);
          }
          if (i == 0) {
#pragma unroll
            for (int z = 0; z < 4 * NJ; ++z) {
              __builtin_amdgcn_sched_group_barrier(0x002, 4, 1);
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            }
          }
          __builtin_amdgcn_s_setprio(0);
          // lane: output rows 16 i + 4 g + q, column 16 j + l%16
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[i][j][q] = __builtin_fmaf(pp[j][q], kWaveWScale ? sc[q] : sc[q] * swj[j], acc[i][j][q]);
          if (i + 1 < MI) {
            xa[0] = cvt8<AF>(n0.x, n0.y, 1.0f);
            xa[1] = cvt8<AF>(n0.z, n0.w, 1.0f);
            xa[2] = cvt8<AF>(n1.x, n1.y, 1.0f);
            xa[3] = cvt8<AF>(n1.z, n1.w, 1.0f);
          }
          // Issue order for the scheduler: the two LDS reads of the next A
          // tile first, then each MFMA followed by two VALU instructions
          // (promotion FMAs and the next tile's conversions).
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
          for (int z = 0; z < 4 * NJ; ++z) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          issue_part(kb, buf, i, MI / 2);
          const int r = a_row0 + 16 * i;
          const float fsa = (MODE == MODE_MX) ? e8m0_to_f32((s_e[buf][0][r] >> (8 * g)) & 0xffu) : 1.0f;
          const u32x4 d0 = lds16(sa_, r * 128 + c0), d1 = lds16(sa_, r * 128 + c1);
          v8bf xa[4];
          xa[0] = cvt8<AF>(d0.x, d0.y, fsa);
          xa[1] = cvt8<AF>(d0.z, d0.w, fsa);
          xa[2] = cvt8<AF>(d1.x, d1.y, fsa);
          xa[3] = cvt8<AF>(d1.z, d1.w, fsa);
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_bf16(xa[s], xb[j][s], acc[i][j]);
        }
      }
    }
    buf = buf + 1 == NS ? 0 : buf + 1;
  }
  // the last step's filler loads still write LDS: drain them before the
  // workgroup can exit
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if constexpr (MX_WORDS) {
    // Block-by-block exact MX: one 32-K block b of the step per instruction,
    // lane group g taking K 32b + 8g .. +7 of its row, the codes expanded with
    // a unit scale (exact), so an instruction's sum P is one block's exact
    // products summed in fp32; P * 2^(eA + eB) joins the accumulator through an
    // exact ldexp (eA of the output row, eB of the output column).  Steps kb ..
    // nkb-1 (the first one's loads are already waited for and published).
    for (bool first = true; mx_wide && kb < nkb; ++kb, first = false) {
      if (!first) sync_step(kb, buf);
      // the main loop issues a step's row blocks from inside its multiply
      // loop; here (including the step the main loop left) they go out whole
      if (kb + NS - 1 < nkb) issue_next(kb, buf, 0, LPW);
      const uint8_t* sa_ = &smem[buf][0];
      const uint8_t* sb_ = &smem[buf][TBM * TBK];
#pragma unroll 1
      for (int b = 0; b < 4; ++b) {
        const int cb = (((2 * b + (g >> 1)) ^ sw_) << 4) + 8 * (g & 1);
        v8bf xbb[NJ];
        int ebj[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const uint2 d = *reinterpret_cast<const uint2*>(sb_ + (b_row0 + 16 * j) * 128 + cb);
          xbb[j] = cvt8<BF>(d.x, d.y, 1.0f);
          ebj[j] = (int)((s_e[buf][0][TBM + b_row0 + 16 * j] >> (8 * b)) & 0xffu) - 127;
        }
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const uint2 d = *reinterpret_cast<const uint2*>(sa_ + (a_row0 + 16 * i) * 128 + cb);
          const v8bf xa = cvt8<AF>(d.x, d.y, 1.0f);
          // UE8M0 words of the tile's output rows 4g .. 4g+3
          const u32x4 wq = *reinterpret_cast<const u32x4*>(&s_e[buf][0][wm * WR + 16 * i + 4 * g]);
          const int ea[4] = {(int)((wq.x >> (8 * b)) & 0xffu) - 127, (int)((wq.y >> (8 * b)) & 0xffu) - 127,
                             (int)((wq.z >> (8 * b)) & 0xffu) - 127, (int)((wq.w >> (8 * b)) & 0xffu) - 127};
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const v4f pb = mfma_bf16(xa, xbb[j], v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][j][q] += __builtin_amdgcn_ldexpf(pb[q], ea[q] + ebj[j]);
          }
        }
      }
      buf = buf + 1 == NS ? 0 : buf + 1;
    }
  }

  // epilogue
  // The quantized outputs: the result quantized to FP8 for the next layer,
  // exactly as the quantizer does it to the fp32 values the DT_F32 output
  // would hold: per row and 128 columns, amax -> s = RN(amax / Vmax) ->
  // sat_rne(RN(v / s)).  Tile scales are stored with a row stride of ldo / 128
  // (the whole output's groups per row), so a column range of the output can
  // be computed as a problem of its own.
  if constexpr ((ODT == ODT_Q_E4M3 || ODT == ODT_Q_E5M2) && kTransposed) {
    // Transposed products: lane l holds row 16 i + l%16, columns 16 j + 4 g + q.
    // The tile starts on a 128-column group; a wave's WC < 128 columns meet at
    // most two groups (slots 0, 1), and a 16-column tile lies in one.  Each
    // wave takes |v| per row over its columns of each group, the waves that
    // share a group combine those partial maxima through LDS, and each lane
    // encodes its four consecutive values of an N tile under their group's
    // scale, one 4-byte store.
    constexpr int QF = ODT == ODT_Q_E4M3 ? FMT_E4M3 : FMT_E5M2;
    static_assert(TBN % 128 == 0 && WC < 128, "tiles on group boundaries, waves narrower than a group");
    constexpr int kSpan = 128 / WC + 1;   // most waves that share a group
    __shared__ float s_pmax[NW][2][WR];
    const int cw = wn * WC, tg0 = cw >> 7;   // the wave's first tile column and its group
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      float pm[2] = {0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float m = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) m = fmaxf(m, fabsf(acc[i][j][q]));
        if (((cw + 16 * j) >> 7) == tg0) pm[0] = fmaxf(pm[0], m);
        else pm[1] = fmaxf(pm[1], m);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        pm[s] = fmaxf(pm[s], __shfl_xor(pm[s], 16));   // over the 4 lanes that hold this row
        pm[s] = fmaxf(pm[s], __shfl_xor(pm[s], 32));
        if (g == 0) s_pmax[w][s][16 * i + (lane & 15)] = pm[s];
      }
    }
    __syncthreads();
    const int64_t nsg = N / 128, srow = p.ldo / 128;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int rl = 16 * i + (lane & 15);   // row within the wave tile
      const int64_t row = m0 + wm * WR + rl;
      float sc[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int tg = tg0 + s;   // a tile group past the tile (slot 1 unused) reads no wave
        const int lo = (tg * 128) / WC, hi = (tg * 128 + 127) / WC < WNW - 1 ? (tg * 128 + 127) / WC : WNW - 1;
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < kSpan; ++k) {
          const int wn2 = lo + k;
          if (wn2 <= hi) amax = fmaxf(amax, s_pmax[wm * WNW + wn2][tg - ((wn2 * WC) >> 7)][rl]);
        }
        sc[s] = group_scale<QF>(amax);
      }
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int cl = cw + 16 * j;   // the N tile's first tile column
        const int64_t grp = (n0 + cl) / 128;
        if (grp >= nsg) continue;     // (N % 128 == 0: a group is stored whole or not at all)
        const float s = ((cl >> 7) == tg0) ? sc[0] : sc[1];
        const float v4[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
        uint32_t codes;
        encode_scaled<QF, 4>(v4, s, &codes);
        *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(p.out) + row * p.ldo + n0 + cl + 4 * g) = codes;
        if (((cl + 4 * g) & 127) == 0) p.out_scales[row * srow + grp] = s;
      }
    }
  } else if constexpr (ODT == ODT_Q_E4M3 || ODT == ODT_Q_E5M2) {
    // Untransposed (lane l holds rows 16 i + 4 g + q, column 16 j + l%16): a
    // 128-column group is the tiles of two neighbouring waves (wn, wn ^ 1).
    constexpr int QF = ODT == ODT_Q_E4M3 ? FMT_E4M3 : FMT_E5M2;
    static_assert(WC == 64 && WNW % 2 == 0, "a 128-column group must be two 64-column wave tiles");
    __shared__ float s_amax[NW][WR];
    if constexpr (MODE == MODE_EPILOGUE) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          int64_t col = n0 + wn * WC + j * 16 + (lane & 15);
          col = col < N ? col : N - 1;   // columns past N hold zeros and are not stored
          const float sbv = swb[p.b_per_row ? col : 0];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            int64_t row = m0 + wm * WR + i * 16 + 4 * g + q;
            row = row < M ? row : M - 1;   // rows past M are not stored
            acc[i][j][q] = acc[i][j][q] * (sxa[p.a_per_row ? row : 0] * sbv);
          }
        }
    }
    float rmax[MI][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) m = fmaxf(m, fabsf(acc[i][j][q]));
        rmax[i][q] = group_max<16>(m);   // over the 16 lanes that hold this row
        if ((lane & 15) == 0) s_amax[w][16 * i + 4 * g + q] = rmax[i][q];
      }
    __syncthreads();
    const int64_t nsg = N / 128, srow = p.ldo / 128;   // scale groups per row, row stride of the scales
    const int64_t grp = (n0 + wn * WC) / 128;          // this wave's group
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int64_t rbase = m0 + wm * WR + i * 16;
      if (rbase >= M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = rbase + 4 * g + q;
        const float amax = fmaxf(rmax[i][q], s_amax[w ^ 1][16 * i + 4 * g + q]);
        const float s = group_scale<QF>(amax);
        const float v4[4] = {acc[i][0][q], acc[i][1][q], acc[i][2][q], acc[i][3][q]};
        uint32_t codes;
        encode_scaled<QF, 4>(v4, s, &codes);
        if (grp < nsg) {
          uint8_t* o = static_cast<uint8_t*>(p.out) + row * p.ldo + n0 + wn * WC + (lane & 15);
#pragma unroll
          for (int j = 0; j < NJ; ++j) o[16 * j] = (uint8_t)(codes >> (8 * j));
          if ((wn & 1) == 0 && (lane & 15) == 0) p.out_scales[row * srow + grp] = s;
        }
      }
    }
  } else if constexpr (kTransposed) {
    // lane: row 16 i + l%16, columns 16 j + 4 g + q (N is a multiple of 16,
    // so an N tile is stored whole or not at all)
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int64_t row = m0 + wm * WR + i * 16 + (lane & 15);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t cbase = n0 + wn * WC + j * 16;
        if (row >= M || cbase >= N) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) store_out<ODT>(p.out, row * p.ldo + cbase + 4 * g + q, acc[i][j][q]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int64_t rbase = m0 + wm * WR + i * 16;
      if (rbase >= M) continue;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t cbase = n0 + wn * WC + j * 16;
        if (cbase >= N) continue;
        const int64_t col = cbase + (lane & 15);
        float sbv = 1.0f;
        if constexpr (MODE == MODE_EPILOGUE) sbv = swb[p.b_per_row ? col : 0];
        if constexpr (MODE == MODE_NV4) sbv = p.ta[0] * p.tb[0];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t row = rbase + 4 * g + q;
          float v = acc[i][j][q];
          if constexpr (MODE == MODE_EPILOGUE) v = v * (sxa[p.a_per_row ? row : 0] * sbv);
          if constexpr (MODE == MODE_NV4) v = v * sbv;
          store_out<ODT>(p.out, row * p.ldo + col, v);
        }
      }
    }
  }
}

// Kernels for the workgroup shapes, 8 waves each: 256x256 and 256x192 (wave
// tiles 128x64, and 64x96 or 128x48, two LDS stages), and 128x256 (wave tiles
// 64x64, three LDS stages) for problems with fewer 256x256 tiles than CUs,
// where the deeper pipeline measured 13% faster and the smaller tile's lower
// arithmetic intensity does not matter; and 64x64 with 4 waves for small
// problems (below).
template <int AF, int BF, int MODE, int ODT, int PATH>
__global__ __launch_bounds__(512, 1) void k_gemm_tiled_256x256(GemmArgs p) {
  gemm_tiled_body<AF, BF, MODE, ODT, PATH, 2, 4, 8, 4, 2>(p);
}
template <int AF, int BF, int MODE, int ODT, int PATH>
__global__ __launch_bounds__(512, 1) void k_gemm_tiled_256x192(GemmArgs p) {
  if constexpr (MODE == MODE_PROMOTE && PATH == PATH_EXACT)
    gemm_tiled_body<AF, BF, MODE, ODT, PATH, 4, 2, 4, 6, 2>(p);   // 64x96 wave tiles, A held, B streamed
  else
    gemm_tiled_body<AF, BF, MODE, ODT, PATH, 2, 4, 8, 3, 2>(p);
}
// (NVFP4 stages 16 scale bytes per row and step: three stages would exceed
// the 160 KiB of LDS, so it runs two.)
template <int AF, int BF, int MODE, int ODT, int PATH>
__global__ __launch_bounds__(512, 1) void k_gemm_tiled_128x256(GemmArgs p) {
  gemm_tiled_body<AF, BF, MODE, ODT, PATH, 2, 4, 4, 4, MODE == MODE_NV4 ? 2 : 3>(p);
}
// 128x384 tiles (wave tiles 64x96, transposed products, two stages): the
// last wave of tiles of an exact-promotion GEMM with quantized output, whose
// 128-column scale groups must not straddle tiles as the 256x192 tiles'
// would; three quarters of a 256x256 tile's work, like those.
template <int AF, int BF, int MODE, int ODT, int PATH>
__global__ __launch_bounds__(512, 1) void k_gemm_tiled_128x384(GemmArgs p) {
  gemm_tiled_body<AF, BF, MODE, ODT, PATH, 2, 4, 4, 6, 2>(p);
}
// 64x64 tiles of 4 waves (32x32 wave tiles, three stages) for problems whose
// 128x256 tiles would leave many CUs idle (128x256x512: one tile, whose
// 128 KiB fp32 result one CU alone would store).  Their conversions per MFMA
// double, so they pay only below a share of the CUs: measured (A/B on one
// box) exact 106 -> 51 us at 256x7168x7168 (56 tiles of 128x256), 64 -> 53 us
// at 1024x4096x4096 (128 tiles); native 67 -> 43 us at 56 tiles but 37 -> 39
// us at 128.
template <int AF, int BF, int MODE, int ODT, int PATH>
__global__ __launch_bounds__(256, 1) void k_gemm_tiled_64x64(GemmArgs p) {
  gemm_tiled_body<AF, BF, MODE, ODT, PATH, 2, 2, 2, 2, 3>(p);
}


// ---------------------------------------------------------------------------
__global__ void k_fill_u32(uint32_t* p, int64_t nwords, uint32_t v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < nwords) p[i] = v;
}

static hipError_t fill_u32(uint32_t* p, int64_t nwords, uint32_t v, hipStream_t st) {
  if (nwords == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((nwords + 255) / 256)), dim3(256), 0, st, p, nwords, v);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* out, int64_t bytes, hipStream_t st) {
  return fill_u32(reinterpret_cast<uint32_t*>(out), bytes / 4, 0u, st);
}

hipError_t launch_fill_f32(float* out, int64_t n, float v, hipStream_t st) {
  return fill_u32(reinterpret_cast<uint32_t*>(out), n, __builtin_bit_cast(uint32_t, v), st);
}

// ---- dispatch over formats, modes, output dtype, path and tile shape ---------
// Tile shapes: 256x256 when that gives at least one tile per CU (with a
// 256x192 remainder, or 128x384 for the quantized outputs, below), else
// 128x256 or 64x64.

// The columns [c0, c0 + n) of the problem as a problem of its own (c0 is a
// multiple of 128, so every scale layout splits at a block boundary).
static GemmArgs column_range(const GemmArgs& p, int64_t c0, int64_t n, int mode, int odt) {
  GemmArgs q = p;
  const bool fp4 = mode == MODE_MX4 || mode == MODE_MX4_PAIRS || mode == MODE_NV4;
  q.b = p.b + c0 * (fp4 ? p.K / 2 : p.K);
  q.N = n;
  q.out = static_cast<uint8_t*>(p.out) + c0 * (odt == DT_F32 ? 4 : (odt == DT_BF16 ? 2 : 1));
  if (odt == ODT_Q_E4M3 || odt == ODT_Q_E5M2) q.out_scales = p.out_scales + c0 / 128;
  if (mode == MODE_PROMOTE) q.sb = static_cast<const float*>(p.sb) + (c0 / 128) * (p.K / 128);
  else if (mode == MODE_MX || mode == MODE_MX4 || mode == MODE_MX4_PAIRS) q.sb = static_cast<const uint8_t*>(p.sb) + c0 * (p.K / 32);
  else if (mode == MODE_NV4) q.sb = static_cast<const uint8_t*>(p.sb) + c0 * (p.K / 16);
  else if (p.b_per_row) q.sb = static_cast<const float*>(p.sb) + c0;
  return q;
}

template <int AF, int BF, int MODE, int ODT, int PATH>
static void tiled_shape(const GemmArgs& p, hipStream_t st) {
  const int64_t cus = num_cus();
  const int64_t ntm = (p.M + 255) / 256;
  const int64_t big_tiles = ntm * ((p.N + 255) / 256);
  if (big_tiles < cus) {
    const int64_t tiles = ((p.M + 127) / 128) * ((p.N + 255) / 256);
    // (Not for the exact MX path: its switch to block-by-block sums is taken
    // per wave, over the wave's rows, so 32-row waves would round some sums
    // differently from the 64-row waves the quantized-output GEMM uses.)
    if constexpr (ODT < ODT_Q_E4M3 && MODE <= MODE_MX && !(MODE == MODE_MX && PATH == PATH_EXACT)) {
      if (PATH == PATH_EXACT ? 5 * tiles <= 3 * cus : 4 * tiles <= cus) {
        const int64_t small = ((p.M + 63) / 64) * ((p.N + 63) / 64);
        hipLaunchKernelGGL((k_gemm_tiled_64x64<AF, BF, MODE, ODT, PATH>), dim3((unsigned)small), dim3(256), 0, st, p);
        return;
      }
    }
    hipLaunchKernelGGL((k_gemm_tiled_128x256<AF, BF, MODE, ODT, PATH>), dim3((unsigned)tiles), dim3(512), 0, st, p);
    return;
  }
  // A tile count that is not a multiple of the CU count leaves part of the
  // last wave of workgroups idle.  When the tile rows divide the CUs, the
  // first N1 columns are done in whole waves of 256x256 tiles and the rest in
  // one wave of 256x192 tiles (three quarters of the work per tile), launched
  // right after: e.g. 4096x7168 runs as 256 + 256 tiles in 1.75 tile-times
  // instead of 448 tiles in 2.
  // The quantized outputs cannot take 256x192 tiles, whose 128-column scale
  // groups would straddle two tiles: exact promotion does its last wave in
  // 128x384 tiles instead (4096x7168x7168: 256 + 256 tiles), other modes do
  // not split.
  // The exact path splits: its steps are bound by the VALU and matrix work,
  // which shrinks with the tile.  The FP8 native path is bound per step by
  // load and LDS latency, so a 256x192 tile takes about as long as a 256x256
  // one; measured at 4096x7168x7168 on rotated inputs, one launch of all 448
  // tiles was 7-8% faster than the split there.  MXFP4 with step-pair scale
  // staging splits too: 2% faster, A/B on one box (MXFP4 with word-by-word
  // staging measured equal either way).
  constexpr bool kQuantOut = ODT == ODT_Q_E4M3 || ODT == ODT_Q_E5M2;
  constexpr bool kSplit = kQuantOut ? (MODE == MODE_PROMOTE && PATH == PATH_EXACT)
                                    : (PATH == PATH_EXACT || MODE == MODE_MX4_PAIRS);
  if constexpr (kSplit) {
    const int64_t wave_cols = cus % ntm == 0 ? (cus / ntm) * 256 : 0;
    const int64_t n1 = wave_cols > 0 ? (p.N / wave_cols) * wave_cols : 0, n2 = p.N - n1;
    const int64_t last = kQuantOut ? ((p.M + 127) / 128) * ((n2 + 383) / 384) : ntm * ((n2 + 191) / 192);
    if (big_tiles % cus != 0 && n1 > 0 && n2 > 0 && last <= cus) {
      const GemmArgs p1 = column_range(p, 0, n1, MODE, ODT), p2 = column_range(p, n1, n2, MODE, ODT);
      hipLaunchKernelGGL((k_gemm_tiled_256x256<AF, BF, MODE, ODT, PATH>), dim3((unsigned)(ntm * (n1 / 256))),
                         dim3(512), 0, st, p1);
      if constexpr (kQuantOut)
        hipLaunchKernelGGL((k_gemm_tiled_128x384<AF, BF, MODE, ODT, PATH>), dim3((unsigned)last), dim3(512), 0,
                           st, p2);
      else
        hipLaunchKernelGGL((k_gemm_tiled_256x192<AF, BF, MODE, ODT, PATH>), dim3((unsigned)last), dim3(512), 0,
                           st, p2);
      return;
    }
  }
  hipLaunchKernelGGL((k_gemm_tiled_256x256<AF, BF, MODE, ODT, PATH>), dim3((unsigned)big_tiles), dim3(512), 0, st, p);
}

template <int AF, int BF, int MODE, int ODT>
static void tiled_path(const GemmArgs& p, int path, hipStream_t st) {
  if (path == PATH_FAST) tiled_shape<AF, BF, MODE, ODT, PATH_FAST>(p, st);
  else tiled_shape<AF, BF, MODE, ODT, PATH_EXACT>(p, st);
}

template <int AF, int BF, int MODE>
static void tiled_odt(const GemmArgs& p, int odt, int path, hipStream_t st) {
  if (odt == DT_F32) tiled_path<AF, BF, MODE, DT_F32>(p, path, st);
  else if (odt == DT_BF16) tiled_path<AF, BF, MODE, DT_BF16>(p, path, st);
  else if (odt == ODT_Q_E4M3) tiled_path<AF, BF, MODE, ODT_Q_E4M3>(p, path, st);
  else tiled_path<AF, BF, MODE, ODT_Q_E5M2>(p, path, st);
}

template <int AF, int BF>
static void tiled_mode(const GemmArgs& p, int mode, int odt, int path, hipStream_t st) {
  if (mode == MODE_EPILOGUE) tiled_odt<AF, BF, MODE_EPILOGUE>(p, odt, path, st);
  else if (mode == MODE_PROMOTE) tiled_odt<AF, BF, MODE_PROMOTE>(p, odt, path, st);
  else tiled_odt<AF, BF, MODE_MX>(p, odt, path, st);
}

hipError_t launch_gemm_fp4(const GemmArgs& p, int mode, int odt, hipStream_t st) {
  // the format template arguments are unused by the FP4 modes
  if (mode == MODE_MX4 && (p.K / 256) % 2 == 0) {
    if (odt == DT_F32) tiled_shape<FMT_E4M3, FMT_E4M3, MODE_MX4_PAIRS, DT_F32, PATH_FAST>(p, st);
    else tiled_shape<FMT_E4M3, FMT_E4M3, MODE_MX4_PAIRS, DT_BF16, PATH_FAST>(p, st);
  } else if (mode == MODE_MX4) {
    if (odt == DT_F32) tiled_shape<FMT_E4M3, FMT_E4M3, MODE_MX4, DT_F32, PATH_FAST>(p, st);
    else tiled_shape<FMT_E4M3, FMT_E4M3, MODE_MX4, DT_BF16, PATH_FAST>(p, st);
  } else {
    if (odt == DT_F32) tiled_shape<FMT_E4M3, FMT_E4M3, MODE_NV4, DT_F32, PATH_EXACT>(p, st);
    else tiled_shape<FMT_E4M3, FMT_E4M3, MODE_NV4, DT_BF16, PATH_EXACT>(p, st);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_tiled(const GemmArgs& p, int afmt, int bfmt, int mode, int odt, int path, hipStream_t st) {
  if (afmt == FMT_E4M3 && bfmt == FMT_E4M3) tiled_mode<FMT_E4M3, FMT_E4M3>(p, mode, odt, path, st);
  else if (afmt == FMT_E4M3) tiled_mode<FMT_E4M3, FMT_E5M2>(p, mode, odt, path, st);
  else if (bfmt == FMT_E4M3) tiled_mode<FMT_E5M2, FMT_E4M3>(p, mode, odt, path, st);
  else tiled_mode<FMT_E5M2, FMT_E5M2>(p, mode, odt, path, st);
  return hipGetLastError();
}

}  // namespace fp8blk
