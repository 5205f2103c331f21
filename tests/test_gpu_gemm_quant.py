"""GPU parity: the GEMM whose result is quantized in its epilogue.

The fused kernel must write exactly the codes and 1x128 tile scales that the
quantizer's definition gives for the fp32 result of the same GEMM: the same
kernel with fp32 output yields those fp32 values (same accumulation order),
the oracle quantizes them on the CPU, and codes and scales must match bit for
bit.  The fp32 values themselves are held to the GEMM tolerance against the
oracle's fp64 reference."""

import numpy as np
import pytest
import torch

import block_scaled_precision_x128_amd as fb
import workloads
from oracle import gemm, quant
from gpu_helpers import (NATIVE_REL_TOL, assert_codes_equal, assert_scales_equal, dev, gemm_check, host,
                         oracle_quantize, say)

pytestmark = pytest.mark.gpu

T, R, TL, BL, MX = (fb.GRAN_TENSOR, fb.GRAN_ROW, fb.GRAN_TILE_1x128, fb.GRAN_BLOCK_128x128, fb.GRAN_MX32)
ACCUMS = [(fb.ACCUM_FP32, gemm.REL_TOL), (fb.ACCUM_NATIVE, NATIVE_REL_TOL)]


def _operands(M, N, K, xg, wg, seed):
    rng = np.random.default_rng(seed)
    wl = workloads.CONFIGS["c3_deepseek_block"]
    x = workloads.draw_x(wl, M, K, rng)
    w = workloads.draw_w(wl, N, K, rng)
    xq, sx = quant.quantize(x, xg, fb.E4M3)
    wq, sw = quant.quantize(w, wg, fb.E4M3)
    return xq, sx, wq, sw


@pytest.mark.parametrize("xg,wg", [(T, T), (R, R), (TL, BL), (MX, MX)])
@pytest.mark.parametrize("out_fmt", [fb.E4M3, fb.E5M2])
def test_fused_quant_matches_quantized_fp32_result(xg, wg, out_fmt):
    # (48, 256): 128x256 tiles with a ragged M; (4096, 4480): 256x256 tiles,
    # with exact promotion (TL, BL) its last 384 columns in 128x384 tiles;
    # (4000, 7168): 256 + 256 tiles, the second wave 128x384 with a ragged M;
    # (4096, 4608): a 128x384 tile with 128 valid columns
    for (M, N, K) in [(48, 256, 384), (272, 384, 640), (4096, 4480, 256), (4000, 7168, 128), (4096, 4608, 128)]:
        xq, sx, wq, sw = _operands(M, N, K, xg, wg, seed=M + N + K + xg)
        a, sa, b, sb = dev(xq), dev(sx), dev(wq), dev(sw)
        for accum, rel in ACCUMS:
            label = f"fused quant pair=({xg},{wg}) out_fmt={out_fmt} {M}x{N}x{K} accum={accum}"
            say(label)
            yf = fb.fp8_gemm_blockscaled(a, fb.E4M3, xg, sa, b, fb.E4M3, wg, sb, fb.DT_F32,
                                         algo=fb.GEMM_TILED, accum=accum)
            codes, scales = fb.fp8_gemm_blockscaled_quant(a, fb.E4M3, xg, sa, b, fb.E4M3, wg, sb, out_fmt,
                                                          accum=accum)
            torch.cuda.synchronize()
            yh = host(yf)
            # 1x128 tiles are per row: large results are checked on a sample of rows
            rows = np.arange(M) if M <= 512 else np.random.default_rng(M).choice(M, 96, replace=False)
            if M * N <= 1 << 18:
                ref, absb = gemm.gemm_ref(xq, sx, xg, fb.E4M3, wq, sw, wg, fb.E4M3)
                gemm_check(yh, fb.DT_F32, ref, absb, label + " fp32 result", rel)
            else:
                # the sampled rows of the fp32 result against the oracle (row scales follow the rows)
                sxr = sx if xg == T else sx[rows]
                ref, absb = gemm.gemm_ref(xq[rows], sxr, xg, fb.E4M3, wq, sw, wg, fb.E4M3)
                gemm_check(yh[rows], fb.DT_F32, ref, absb, label + " fp32 result (sampled rows)", rel)
            want_q, want_s = oracle_quantize(yh[rows], TL, out_fmt)
            assert_scales_equal(host(scales)[rows], want_s, label)
            assert_codes_equal(host(codes)[rows], want_q, label + " codes", yh[rows])


def test_fused_quant_k_zero():
    say("fused quant K=0")
    a = torch.empty((32, 0), dtype=torch.uint8, device="cuda")
    b = torch.empty((256, 0), dtype=torch.uint8, device="cuda")
    one = torch.ones(1, device="cuda")
    codes = torch.full((32, 256), 7, dtype=torch.uint8, device="cuda")
    scales = torch.zeros((32, 2), device="cuda")
    fb.fp8_gemm_blockscaled_quant(a, fb.E4M3, T, one, b, fb.E4M3, T, one, fb.E4M3, codes=codes, scales=scales)
    torch.cuda.synchronize()
    assert int(codes.sum()) == 0
    assert host(scales).tolist() == [[1.0, 1.0]] * 32
