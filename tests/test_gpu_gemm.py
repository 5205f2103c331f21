"""GPU parity: block-scaled FP8 GEMM against the oracle's fp64 reference.

Operands are quantized by the oracle on the CPU and the same codes and scales
go to both sides.  Bound (default fp32 accumulation): |out - Ref| <= 1e-4 *
sum_k |x_k w_k| per element, plus half a bf16 ulp of the output for bf16
outputs.  The FP8 instructions' own accumulation (accum=NATIVE) is held to
its documented 1e-3 bound."""

import numpy as np
import pytest
import torch

import block_scaled_precision_x128_amd as fb
import workloads
from oracle import formats, gemm, quant
from gpu_helpers import NATIVE_REL_TOL, dev, gemm_check, host, say

pytestmark = pytest.mark.gpu

T, R, TL, BL, MX = (fb.GRAN_TENSOR, fb.GRAN_ROW, fb.GRAN_TILE_1x128, fb.GRAN_BLOCK_128x128, fb.GRAN_MX32)
PAIRS = [(T, T), (T, R), (R, T), (R, R), (TL, BL), (MX, MX)]
FMT_PAIRS = [(fb.E4M3, fb.E4M3), (fb.E4M3, fb.E5M2), (fb.E5M2, fb.E4M3), (fb.E5M2, fb.E5M2)]


def _operands(M, N, K, xg, wg, xf, wf, seed):
    rng = np.random.default_rng(seed)
    wl = workloads.CONFIGS["c3_deepseek_block"]
    x = workloads.draw_x(wl, M, K, rng)
    if wg == MX:
        w = workloads.draw_w(workloads.CONFIGS["c5_mxfp8_mix"], N, K, rng)
    else:
        w = workloads.draw_w(wl, N, K, rng)
    xq, sx = quant.quantize(x, xg, xf)
    wq, sw = quant.quantize(w, wg, wf)
    return xq, sx, wq, sw


ACCUMS = [(fb.ACCUM_FP32, gemm.REL_TOL), (fb.ACCUM_NATIVE, NATIVE_REL_TOL)]


def _run(xq, sx, xg, xf, wq, sw, wg, wf, odt, algo, accum=fb.ACCUM_FP32):
    out = fb.fp8_gemm_blockscaled(dev(xq), xf, xg, dev(sx), dev(wq), wf, wg, dev(sw), odt, algo=algo,
                                  accum=accum)
    torch.cuda.synchronize()
    return host(out)


def _shapes(wg):
    if wg == BL:
        return [(16, 128, 128), (48, 256, 384), (272, 384, 640), (128, 256, 1024)]
    return [(16, 16, 128), (48, 80, 256), (272, 400, 640), (128, 256, 1024)]


@pytest.mark.parametrize("xg,wg", PAIRS)
@pytest.mark.parametrize("xf,wf", FMT_PAIRS)
def test_gemm_small_ragged(xg, wg, xf, wf):
    for (M, N, K) in _shapes(wg):
        xq, sx, wq, sw = _operands(M, N, K, xg, wg, xf, wf, seed=M * 31 + N + K)
        ref, absb = gemm.gemm_ref(xq, sx, xg, xf, wq, sw, wg, wf)
        algos = [fb.GEMM_TILED] + ([fb.GEMM_SKINNY] if M <= 64 else [])
        for algo in algos:
            for accum, rel in ACCUMS:
                for odt in (fb.DT_F32, fb.DT_BF16):
                    label = f"pair=({xg},{wg}) fmt=({xf},{wf}) {M}x{N}x{K} algo={algo} accum={accum} odt={odt}"
                    say("gemm", label)
                    out = _run(xq, sx, xg, xf, wq, sw, wg, wf, odt, algo, accum)
                    gemm_check(out, odt, ref, absb, label, rel)


def test_gemm_integer_codes_exact():
    """Codes of small integers with unit scales: the fp32 result is an exact
    integer matmul (sums below 2^24), so it must match bit for bit."""
    rng = np.random.default_rng(3)
    M, N, K = 64, 128, 512
    xi = rng.integers(-16, 17, (M, K))
    wi = rng.integers(-16, 17, (N, K))
    xq = formats.encode(xi.astype(np.float64), fb.E4M3)
    wq = formats.encode(wi.astype(np.float64), fb.E4M3)
    one = np.ones(1, np.float32)
    want = (xi @ wi.T).astype(np.float32)
    for algo in (fb.GEMM_TILED, fb.GEMM_SKINNY):
        for accum, _ in ACCUMS:
            say("gemm integer exact", algo, accum)
            out = _run(xq, one, T, fb.E4M3, wq, one, T, fb.E4M3, fb.DT_F32, algo, accum)
            assert np.array_equal(out, want)


def test_gemm_mx_scales_are_per_32_block():
    """A different UE8M0 exponent for every 32-K block and row: the result
    must apply each block's own power of two (checks which lanes' scales the
    scaled MFMA applies to which K elements)."""
    rng = np.random.default_rng(4)
    M, N, K = 32, 32, 256
    xq = formats.encode(rng.integers(-3, 4, (M, K)).astype(np.float64), fb.E4M3)
    wq = formats.encode(rng.integers(-3, 4, (N, K)).astype(np.float64), fb.E5M2)
    ex = (127 + rng.integers(-3, 4, (M, K // 32))).astype(np.uint8)
    ew = (127 + rng.integers(-3, 4, (N, K // 32))).astype(np.uint8)
    ref, absb = gemm.gemm_ref(xq, ex, MX, fb.E4M3, wq, ew, MX, fb.E5M2)
    for algo in (fb.GEMM_TILED, fb.GEMM_SKINNY):
        for accum, rel in ACCUMS:
            say("gemm mx blocks", algo, accum)
            out = _run(xq, ex, MX, fb.E4M3, wq, ew, MX, fb.E5M2, fb.DT_F32, algo, accum)
            gemm_check(out, fb.DT_F32, ref, absb, f"mx per-block algo={algo} accum={accum}", rel)


def test_gemm_skinny_matches_tiled():
    M, N, K = 32, 1024, 2048
    xq, sx, wq, sw = _operands(M, N, K, TL, BL, fb.E4M3, fb.E4M3, seed=8)
    say("gemm skinny vs tiled")
    ref, absb = gemm.gemm_ref(xq, sx, TL, fb.E4M3, wq, sw, BL, fb.E4M3)
    for accum, rel in ACCUMS:
        a = _run(xq, sx, TL, fb.E4M3, wq, sw, BL, fb.E4M3, fb.DT_F32, fb.GEMM_TILED, accum)
        b = _run(xq, sx, TL, fb.E4M3, wq, sw, BL, fb.E4M3, fb.DT_F32, fb.GEMM_SKINNY, accum)
        gemm_check(a, fb.DT_F32, ref, absb, f"tiled accum={accum}", rel)
        gemm_check(b, fb.DT_F32, ref, absb, f"skinny accum={accum}", rel)
        assert np.all(np.abs(a.astype(np.float64) - b) <= 2 * rel * absb)


@pytest.mark.parametrize("xg,wg", PAIRS)
def test_gemm_skinny_partial_tiles(xg, wg):
    """The skinny kernel gives each workgroup R = ceil(N / grid) rows of W, so a
    16-column tile is often only partly inside a workgroup's range and a
    range may straddle a 128-row W scale block: every column must still come
    out right (M = 16, 48 and 64 use 5, 3 and 2 tiles per workgroup; N = 20608
    needs two workgroups per compute unit)."""
    for (M, N, K) in [(16, 4480, 512), (48, 4480, 384), (64, 4480, 256), (16, 20608, 256)]:
        xq, sx, wq, sw = _operands(M, N, K, xg, wg, fb.E4M3, fb.E5M2, seed=N + M)
        ref, absb = gemm.gemm_ref(xq, sx, xg, fb.E4M3, wq, sw, wg, fb.E5M2)
        for accum, rel in ACCUMS:
            label = f"skinny partial tiles pair=({xg},{wg}) {M}x{N}x{K} accum={accum}"
            say("gemm", label)
            out = _run(xq, sx, xg, fb.E4M3, wq, sw, wg, fb.E5M2, fb.DT_F32, fb.GEMM_SKINNY, accum)
            gemm_check(out, fb.DT_F32, ref, absb, label, rel)


@pytest.mark.parametrize("xg,wg", [(R, R), (TL, BL), (MX, MX)])
def test_gemm_tiled_column_split(xg, wg):
    """M = 4096, N = 4480: 16 x 18 = 288 tiles of 256x256 do not fill whole
    waves of 256 CUs, so the kernel runs the first 4096 columns as 256x256
    tiles and the last 384 as 256x192 tiles.  Every column next to the split,
    the last columns and random positions are checked."""
    M, N, K = 4096, 4480, 256
    xq, sx, wq, sw = _operands(M, N, K, xg, wg, fb.E4M3, fb.E4M3, seed=44)
    rng = np.random.default_rng(45)
    cols = np.concatenate([np.arange(4032, 4160), np.arange(N - 64, N), rng.integers(0, N, 2048)])
    mi = np.concatenate([rng.integers(0, M, cols.size)])
    um, mi_idx = np.unique(mi, return_inverse=True)
    un, ni_idx = np.unique(cols, return_inverse=True)
    ref, absb = gemm.gemm_ref_pairs(gemm.dequant_rows(xq[um], sx, xg, fb.E4M3, um),
                                    gemm.dequant_rows(wq[un], sw, wg, fb.E4M3, un), mi_idx, ni_idx)
    for accum, rel in ACCUMS:
        label = f"column split pair=({xg},{wg}) accum={accum}"
        say("gemm", label)
        out = _run(xq, sx, xg, fb.E4M3, wq, sw, wg, fb.E4M3, fb.DT_F32, fb.GEMM_TILED, accum)
        gemm_check(out[mi, cols], fb.DT_F32, ref, absb, label, rel)


def test_gemm_k_zero_writes_zeros():
    say("gemm K=0")
    a = torch.empty((32, 0), dtype=torch.uint8, device="cuda")
    b = torch.empty((64, 0), dtype=torch.uint8, device="cuda")
    s = torch.ones(1, dtype=torch.float32, device="cuda")
    out = torch.full((32, 64), 7.0, dtype=torch.float32, device="cuda")
    fb.fp8_gemm_blockscaled(a, fb.E4M3, T, s, b, fb.E4M3, T, s, fb.DT_F32, out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("xg,wg", [(R, R), (TL, BL), (MX, MX)])
def test_gemm_large_tiles_short_k_and_ragged_m(xg, wg):
    """256x256 tiles (and the 256x192 column split) on one K step, where the
    step's in-loop loads are all fillers past the descriptors, and on three
    steps with a ragged last tile row (M = 4000: 160 of its 256 rows valid);
    and 128x256 tiles on every path at 2560x2048 (160 tiles, too many for the
    64x64 tiles of smaller problems).  Every column of the last tile row, the
    first rows of every tile row and random rows are checked against the
    oracle."""
    for (M, N, K) in [(4096, 4480, 128), (4000, 4480, 384), (4000, 4096, 384), (2560, 2048, 640)]:
        xq, sx, wq, sw = _operands(M, N, K, xg, wg, fb.E4M3, fb.E4M3, seed=M + N + K + xg)
        rng = np.random.default_rng(K + xg)
        rows = np.unique(np.concatenate([np.arange(3840, M), np.arange(0, M, 256), rng.integers(0, M, 64)]))
        xr = gemm.dequant_rows(xq[rows], sx, xg, fb.E4M3, rows)
        wd = gemm.dequant_operand(wq, sw, wg, fb.E4M3)
        ref, absb = xr @ wd.T, np.abs(xr) @ np.abs(wd).T
        for accum, rel in ACCUMS:
            for odt in (fb.DT_F32, fb.DT_BF16):
                label = f"large tiles pair=({xg},{wg}) {M}x{N}x{K} accum={accum} odt={odt}"
                say("gemm", label)
                out = _run(xq, sx, xg, fb.E4M3, wq, sw, wg, fb.E4M3, odt, fb.GEMM_TILED, accum)
                gemm_check(out[rows], odt, ref, absb, label, rel)
