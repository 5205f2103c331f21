/*
 * fp8blk_probe.h -- measurement probes shipped with libfp8blk (C ABI).
 *
 * These are not part of the FP8 method.  They measure the ceilings that the
 * library's kernels are judged against on the machine they run on, beside the
 * published peaks: the matrix-core rate of back-to-back independent MFMAs (the
 * FLOP ceiling of a GEMM main loop, "The FP8 Family", "What Hopper actually
 * gives you": compute roof and ridge point), a plain streaming read and a plain
 * device copy (the bandwidth ceilings of the quantize, dequantize and decode
 * paths, "FP8 Serving", "What FP8 actually buys": decode speed follows the
 * bytes read).
 *
 * Conventions are those of fp8blk.h: device pointers owned by the caller,
 * work enqueued on `stream` without synchronizing, arguments checked on the
 * host first (FP8_ERR_* from fp8blk.h), nothing thrown across the ABI.
 */
#ifndef FP8BLK_PROBE_H
#define FP8BLK_PROBE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core probe kinds. */
typedef enum {
  FP8BLK_PROBE_MFMA_BF16 = 0, /* v_mfma_f32_16x16x32_bf16: 16384 FLOP per instruction        */
  FP8BLK_PROBE_MFMA_FP8 = 1   /* v_mfma_f32_16x16x128_f8f6f4 on E4M3: 65536 FLOP per instruction */
} fp8blk_probe_mfma_t;

/* Floats of `sink` that fp8blk_probe_mfma writes: one per thread of its grid. */
size_t fp8blk_probe_mfma_sink_floats(int waves_per_simd);

/* Back-to-back MFMAs with no memory traffic: one workgroup per compute unit
 * with 4 * waves_per_simd waves (waves_per_simd in 1..2), each wave running
 * `iters` rounds of 8 independent accumulator chains.  Writes one float per
 * thread to sink (fp8blk_probe_mfma_sink_floats() floats) so the work is kept;
 * *flops receives the FLOP count of the launch (2 M N K per instruction times
 * the instructions issued).  Returns FP8_ERR_ENUM for a bad kind,
 * FP8_ERR_SHAPE for waves_per_simd outside 1..2 or iters < 1, FP8_ERR_NULL for
 * a NULL sink or flops. */
int fp8blk_probe_mfma(int kind, int waves_per_simd, int iters, float* sink, double* flops, hipStream_t stream);

/* Floats of `sink` that fp8blk_probe_read writes. */
size_t fp8blk_probe_read_sink_floats(void);

/* Streaming read of `bytes` bytes at src (16-byte aligned, bytes % 16 == 0):
 * every byte is loaded once with 16-byte loads, each workgroup streaming one
 * contiguous chunk with eight loads in flight per thread, and folded into one
 * word per thread written to sink (fp8blk_probe_read_sink_floats() floats). */
int fp8blk_probe_read(const void* src, int64_t bytes, float* sink, hipStream_t stream);

/* Device copy of `bytes` bytes from src to dst (both 16-byte aligned, bytes %
 * 16 == 0, not overlapping) with 16-byte non-temporal loads and stores, one
 * contiguous chunk per workgroup, eight loads in flight per thread. */
int fp8blk_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8BLK_PROBE_H */
