// Device helpers shared by the GEMM kernels (gemm.hip, gemm_skinny.hip):
// matrix-core wrappers, FP8 -> bf16 operand expansion, buffer-descriptor
// loads and output stores.  See gemm.hip for the operand layouts.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace fp8blk {


typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr uint32_t kUnitScale = 0x7f7f7f7fu;  // E8M0 127 = 2^0 in every byte
// Word 3 of a gfx9 buffer descriptor for raw byte-addressed access.
constexpr int kBufferFlags = 0x00020000;

// 16-byte load through a buffer descriptor; offsets at or past the
// descriptor's size read as zero.
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t rs, int voff) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0);
  return u32x4{(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
}

// LDS tiles are stored as 128-byte rows of eight 16-byte chunks; chunk c of
// row r is kept at position c ^ lds_swz(r).  A fragment read has each group of
// 16 lanes fetch one chunk from each of 16 consecutive rows; with this swizzle
// those reads are free of LDS bank conflicts on gfx950 (measured with
// SQ_LDS_BANK_CONFLICT; the plain r & 7 and (r >> 1) & 7 swizzles both stall
// 4 cycles per ds_read_b128).
__device__ __forceinline__ int lds_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Raw buffer descriptor over [base, base + bytes) (bytes <= 0: empty, every
// load reads zeros).  The arguments must be wave-uniform; they are moved to
// scalar registers explicitly so that the descriptor can feed the scalar
// operand of the assembly loads below.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int nb = __builtin_amdgcn_readfirstlane((int)(bytes > 0 ? bytes : 0));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), 0, nb, kBufferFlags);
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p);
}

// Per-lane load of SIZE (16 or 4) bytes at buffer offset voff, written by the
// load unit straight into LDS at lds_base + SIZE * lane (offsets at or past
// the descriptor's size write zeros).  Issued as assembly on purpose: the
// compiler cannot tell which LDS stage such a load targets, so for its own
// load-to-LDS instruction it waits for every one in flight before any later
// LDS read, which would serialize a double-buffered pipeline.  The caller
// orders these loads with s_waitcnt vmcnt(0) and a workgroup barrier before
// any wave reads the stage they fill.  M0 is written here and every load to
// LDS in this library goes through this function, so no compiler-set M0 value
// is relied on across it.
template <int SIZE>
__device__ __forceinline__ void dma_to_lds(__amdgpu_buffer_rsrc_t rs, uint32_t lds_base, int voff) {
  static_assert(SIZE == 16 || SIZE == 4, "16- or 4-byte loads");
  // wave-uniform by contract; read from the first lane so that the compiler
  // places it in a scalar register even where it cannot prove uniformity
  lds_base = __builtin_amdgcn_readfirstlane(lds_base);
  if constexpr (SIZE == 16)
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "s"(lds_base)
                 : "memory");
  else
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "s"(lds_base)
                 : "memory");
}

// dma_to_lds<16> at buffer offset voff + soff (soff wave-uniform), the sum
// formed inside the same assembly block: a kernel that issues many such loads
// from per-lane bases it keeps for the whole loop then holds no per-load
// offset registers (the compiler would otherwise keep each sum live across
// the loop).  Offsets add modulo 2^32; a sum at or past the descriptor's size
// writes zeros.
__device__ __forceinline__ void dma16_to_lds_add(__amdgpu_buffer_rsrc_t rs, uint32_t lds_base, int voff, int soff) {
  lds_base = __builtin_amdgcn_readfirstlane(lds_base);   // wave-uniform by contract (as dma_to_lds)
  soff = __builtin_amdgcn_readfirstlane(soff);
  int sum;
  asm volatile("v_add_u32 %0, %1, %2\n\ts_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %4, 0 offen lds"
               : "=&v"(sum)
               : "s"(soff), "v"(voff), "s"(lds_base), "s"(rs)
               : "memory");
}

template <int AF, int BF>
__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, AF, BF, 0, sa, 0, sb);
}

// FP4 (E2M1) x FP4 with UE8M0 block scales: each operand is 16 bytes (32
// codes) per lane; the upper half of the 8-register operand is not read.
__device__ __forceinline__ v4f mfma_fp4(const u32x4& a, const u32x4& b, const v4f& c, int sa, int sb) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
}

__device__ __forceinline__ v4f mfma_bf16(const v8bf& a, const v8bf& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_f16(const v8h& a, const v8h& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8i join(const u32x4& lo, const u32x4& hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// 2 FP8 codes (16-bit word `hi` of w) -> 2 bf16, multiplied by `scale` (a power of two or 1).
template <int FMT>
__device__ __forceinline__ v2bf cvt2(uint32_t w, float scale, bool hi) {
  if constexpr (FMT == FMT_E4M3) {
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, true)
              : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, false);
  } else {
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, scale, true)
              : __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, scale, false);
  }
}

// Eight E2M1 codes to fp16, times an E4M3 microscale m (given as the fp16
// pair {m, m}): exact converts (scale 1) and a packed fp16 multiply, exact too
// since a code times an E4M3 value has at most 6 significant bits and lies in
// [2^-10, 2688].
__device__ __forceinline__ v8h cvt8_fp4_f16(uint32_t w, v2h m) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * m;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * m;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * m;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * m;
  return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// The E4M3 microscales in bytes 2h and 2h+1 of w as fp16 pairs {m, m}: the
// hardware convert with a unit scale, exact (every E4M3 value, NaN included,
// is an fp16 value).
__device__ __forceinline__ void e4m3_pair_f16(uint32_t w, int h, v2h& m0, v2h& m1) {
  const v2h m = h ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
                  : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  m0 = v2h{m[0], m[0]};
  m1 = v2h{m[1], m[1]};
}

// The 8 codes of dwords (d0, d1) -> one K=32 bf16 operand.
template <int FMT>
__device__ __forceinline__ v8bf cvt8(uint32_t d0, uint32_t d1, float scale) {
  const v2bf p0 = cvt2<FMT>(d0, scale, false), p1 = cvt2<FMT>(d0, scale, true);
  const v2bf p2 = cvt2<FMT>(d1, scale, false), p3 = cvt2<FMT>(d1, scale, true);
  return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Whether folding the MX block scale 2^(byte - 127) into the bf16 expansion
// of FMT codes is exact and stays in bf16's normal range: every nonzero code
// times 2^e lies in [2^-126, 2^128) when e is in [-117, 119] (E4M3: codes
// 2^-9 .. 448) or [-110, 112] (E5M2: codes 2^-16 .. 57344).  Outside that
// range the GEMMs apply 2^(eA + eB) to each 32-K block's fp32 sum instead.
template <int FMT>
__device__ __forceinline__ bool mx_fold_exact(uint32_t byte) {
  constexpr uint32_t lo = FMT == FMT_E4M3 ? 127 - 117 : 127 - 110;
  constexpr uint32_t hi = FMT == FMT_E4M3 ? 127 + 119 : 127 + 112;
  return byte - lo <= hi - lo;
}

// 2^(byte - 127) as fp32 (byte 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t byte) {
  return byte ? __uint_as_float(byte << 23) : __uint_as_float(0x00400000u);
}

template <int ODT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
  if constexpr (ODT == DT_F32) {
    reinterpret_cast<float*>(out)[idx] = v;
  } else {
    const __bf16 h = (__bf16)v;
    reinterpret_cast<uint16_t*>(out)[idx] = __builtin_bit_cast(uint16_t, h);
  }
}

// Buffer offset that lies past every descriptor's range: loads through it
// return zeros without touching memory.
constexpr int kOutOfRange = 0x7ff00000;

// Byte offset a + b modulo 2^32, as the buffer unit adds them: a valid offset
// plus kOutOfRange can pass INT_MAX, and stays past every descriptor's range.
__device__ __forceinline__ int off_add(int a, int b) { return (int)((uint32_t)a + (uint32_t)b); }

// Compute units of the current device (cached per device).
inline int num_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    cus[dev] = (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) ? v : 256;
  }
  return cus[dev];
}

}  // namespace fp8blk
