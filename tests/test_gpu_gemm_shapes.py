"""GPU parity of the FP8 GEMM across the kernel choices the tiled path makes by
problem size: 64x64 tiles for small problems (on the exact path up to
mid-size ones), 128x256 tiles, 256x256 tiles with the 256x192 column split, and
256x256 tiles with a partial last wave and a ragged last tile row.  Every scale
pair, both accumulations, bf16 output; sampled rows (the first and last rows
and random ones) are checked over all columns against the oracle."""

import numpy as np
import pytest

import block_scaled_precision_x128_amd as fb
import workloads
from oracle import gemm, quant
from gpu_helpers import NATIVE_REL_TOL, dev, gemm_check, host, say

pytestmark = pytest.mark.gpu

T, R, TL, BL, MX = (fb.GRAN_TENSOR, fb.GRAN_ROW, fb.GRAN_TILE_1x128, fb.GRAN_BLOCK_128x128, fb.GRAN_MX32)

# (M, N, K): 64x64 tiles on both paths; 64x64 (exact) or 128x256 (native);
# 128x256 on both; the column split; a partial last wave of 256x256 tiles
SHAPES = [(80, 384, 256), (400, 1536, 512), (1040, 2304, 384), (2064, 3072, 256), (4096, 4224, 256),
          (4112, 4096, 128)]


@pytest.mark.parametrize("xg,wg", [(T, T), (R, R), (TL, BL), (MX, MX)])
def test_gemm_across_tile_classes(xg, wg):
    wl = workloads.CONFIGS["c3_deepseek_block"]
    for (M, N, K) in SHAPES:
        rng = np.random.default_rng(M * 7 + N + K + xg)
        x = workloads.draw_x(wl, M, K, rng)
        w = workloads.draw_w(workloads.CONFIGS["c5_mxfp8_mix"] if wg == MX else wl, N, K, rng)
        xq, sx = quant.quantize(x, xg, fb.E4M3)
        wq, sw = quant.quantize(w, wg, fb.E4M3)
        rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 40)]))
        xr = gemm.dequant_rows(xq[rows], sx, xg, fb.E4M3, rows)
        wd = gemm.dequant_operand(wq, sw, wg, fb.E4M3)
        ref, absb = xr @ wd.T, np.abs(xr) @ np.abs(wd).T
        a, sa, b, sb = dev(xq), dev(sx), dev(wq), dev(sw)
        for accum, rel in ((fb.ACCUM_FP32, gemm.REL_TOL), (fb.ACCUM_NATIVE, NATIVE_REL_TOL)):
            label = f"tile classes pair=({xg},{wg}) {M}x{N}x{K} accum={accum}"
            say("gemm", label)
            out = fb.fp8_gemm_blockscaled(a, fb.E4M3, xg, sa, b, fb.E4M3, wg, sb, fb.DT_BF16, algo=fb.GEMM_TILED,
                                          accum=accum)
            gemm_check(host(out)[rows], fb.DT_BF16, ref, absb, label, rel)
