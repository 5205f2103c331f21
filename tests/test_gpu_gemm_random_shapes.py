"""GPU parity of the FP8 GEMM, plain and with quantized output, on seeded
random shapes.  Half are drawn freely within the entry points' limits
(M % 16, N % 128, K % 128); half sit where the tiled path changes its launch:
grids of 256x256 tiles whose tile rows divide the CU count, with a column
count that leaves a partial last wave, which the path splits off into
narrower tiles (a ragged last tile row included); six more have M <= 64,
where the automatic choice is the skinny kernel.  So the tile classes, both
kinds of column split and the skinny kernel are met at shapes that no other
test names.

Each shape draws its scale pair, operand formats and output dtype; both
accumulations run.  Sampled rows (first, last and random ones) are checked over
all columns against the oracle's fp64 GEMM; the quantized output's codes and
1x128 scales must equal, bit for bit, the oracle's quantization of the fp32
result of the same kernel."""

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
PAIRS = [(T, T), (R, R), (TL, BL), (MX, MX)]
ACCUMS = [(fb.ACCUM_FP32, gemm.REL_TOL), (fb.ACCUM_NATIVE, NATIVE_REL_TOL)]


def _shapes(n: int, seed: int):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        if i % 2 == 0:
            M = 16 * int(rng.integers(1, 320))
            N = 128 * int(rng.integers(1, 48))
            K = 128 * int(rng.integers(1, 9))
        else:
            ntm = int(rng.choice([4, 8, 16, 32]))              # 256-row tile rows, a divisor of 256 CUs
            M = 256 * ntm - 16 * int(rng.integers(0, 16))
            wave_cols = (256 // ntm) * 256                     # columns of one full wave of 256x256 tiles
            N = wave_cols + 128 * int(rng.integers(1, wave_cols // 128))
            K = 128 * int(rng.integers(1, 3))
        out.append((M, N, K))
    return out


def _skinny_shapes(n: int, seed: int):
    # M <= 64: the automatic choice streams W through the skinny kernel
    rng = np.random.default_rng(seed)
    return [(16 * int(rng.integers(1, 5)), 128 * int(rng.integers(1, 160)), 128 * int(rng.integers(1, 17)))
            for _ in range(n)]


SHAPES = _shapes(24, seed=20261203) + _skinny_shapes(6, seed=20261204)


@pytest.mark.parametrize("idx", range(len(SHAPES)))
def test_gemm_random_shape(idx):
    M, N, K = SHAPES[idx]
    rng = np.random.default_rng(1000 + idx)
    xg, wg = PAIRS[int(rng.integers(len(PAIRS)))]
    af, bf = (int(rng.choice([fb.E4M3, fb.E5M2])) for _ in range(2))
    odt = int(rng.choice([fb.DT_F32, fb.DT_BF16]))
    qfmt = int(rng.choice([fb.E4M3, fb.E5M2]))
    wl = workloads.CONFIGS["c3_deepseek_block"]
    x = workloads.draw_x(wl, M, K, rng)
    w = workloads.draw_w(workloads.CONFIGS["c5_mxfp8_mix"] if wg == MX else wl, N, K, rng)
    xq, sx = quant.quantize(x, xg, af)
    wq, sw = quant.quantize(w, wg, bf)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 24)]))
    xr = gemm.dequant_rows(xq[rows], sx, xg, af, rows)
    wd = gemm.dequant_operand(wq, sw, wg, bf)
    ref, absb = xr @ wd.T, np.abs(xr) @ np.abs(wd).T
    a, sa, b, sb = dev(xq), dev(sx), dev(wq), dev(sw)
    for accum, rel in ACCUMS:
        label = (f"random shape {idx}: {M}x{N}x{K} pair=({xg},{wg}) fmts=({af},{bf}) out_dt={odt} "
                 f"accum={accum}")
        say("gemm", label)
        out = fb.fp8_gemm_blockscaled(a, af, xg, sa, b, bf, wg, sb, odt, accum=accum)
        gemm_check(host(out)[rows], odt, ref, absb, label, rel)
        del out
        say("gemm quantized output", label, f"out_fmt={qfmt}")
        yf = fb.fp8_gemm_blockscaled(a, af, xg, sa, b, bf, wg, sb, fb.DT_F32, algo=fb.GEMM_TILED, accum=accum)
        codes, scales = fb.fp8_gemm_blockscaled_quant(a, af, xg, sa, b, bf, wg, sb, qfmt, accum=accum)
        torch.cuda.synchronize()
        yh = host(yf)[rows]
        gemm_check(yh, fb.DT_F32, ref, absb, label + " tiled fp32", rel)
        want_q, want_s = oracle_quantize(yh, TL, qfmt)
        assert_scales_equal(host(scales)[rows], want_s, label)
        assert_codes_equal(host(codes)[rows], want_q, label + " codes", yh)
        del yf, codes, scales
