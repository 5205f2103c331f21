"""GPU parity at the edges of the block-scaled FP8 GEMM.

* MX32 at the ends of the UE8M0 range.  The exact path folds a block's 2^e
  into each operand's bf16 expansion while that is exact and finite; steps
  whose exponents leave that range are summed block by block (each 32-K block's
  exact products in fp32, scaled by 2^(eA + eB)).  The products tested here
  are ordinary fp32 numbers even though one operand's scale is 2^-127 .. 2^-124
  and the other's 2^124 .. 2^127, so the 1e-4 * sum|x w| bound applies.  Codes
  cover every finite code of the format.  Both kernels (tiled, skinny), every
  tiled tile shape (64x64, 128x256, 256x256, the 256x192 column split) and both
  orientations; steps switching from foldable to unfoldable exponents midway.
* Operands the quantizer itself makes at those ends: blocks with amax near the
  fp32 maximum (e = 120 for E4M3, codes whose value exceeds fp32's range on its
  own) and blocks with amax below 448 * 2^-127 (byte 0 with nonzero codes).
* The plain entry point fp8_gemm_blockscaled, called through ctypes with raw
  device pointers.
* The FP8 matrix cores' own accumulation (reading G17): a crafted group of
  products in which the largest is 2^10 and the others are small.  The exact
  path returns the exact sum; the native path loses the small products' low
  bits, beyond 1e-4 of the sum but within the documented 7 * 2^-13 of the
  group's largest product.
"""

import ctypes

import numpy as np
import pytest
import torch

import block_scaled_precision_x128_amd as fb
import workloads
from oracle import formats, gemm, quant
from gpu_helpers import NATIVE_REL_TOL, dev, gemm_check, host, say

pytestmark = pytest.mark.gpu

MX = fb.GRAN_MX32


def _finite_codes(fmt):
    c = np.arange(256)
    v = formats.decode(c.astype(np.uint8), fmt)
    return c[np.isfinite(v)].astype(np.uint8)


def _crafted(rows, K, fmt, byte_lo, byte_hi, rng, normal_blocks=0):
    """Random finite codes of fmt; UE8M0 bytes drawn from [byte_lo, byte_hi]
    except the first `normal_blocks` 32-K blocks of every row (bytes 120..134)."""
    q = rng.choice(_finite_codes(fmt), size=(rows, K))
    s = rng.integers(byte_lo, byte_hi + 1, size=(rows, K // 32)).astype(np.uint8)
    s[:, :normal_blocks] = rng.integers(120, 135, size=(rows, normal_blocks))
    return q, s


def _check(xq, sx, xf, wq, sw, wf, algo, accum, label, rows=None):
    out = fb.fp8_gemm_blockscaled(dev(xq), xf, MX, dev(sx), dev(wq), wf, MX, dev(sw), fb.DT_F32, algo=algo,
                                  accum=accum)
    torch.cuda.synchronize()
    o = host(out)
    if rows is not None:
        o, xq, sx = o[rows], xq[rows], sx[rows]
    ref, absb = gemm.gemm_ref(xq, sx, MX, xf, wq, sw, MX, wf)
    assert np.isfinite(ref).all()
    gemm_check(o, fb.DT_F32, ref, absb, label, gemm.REL_TOL if accum == fb.ACCUM_FP32 else NATIVE_REL_TOL)


SHAPES = [(16, 256, 1024, fb.GEMM_SKINNY),     # skinny kernel
          (128, 256, 1024, fb.GEMM_TILED),     # 64x64 tiles (tiny problem)
          (2048, 2048, 1024, fb.GEMM_TILED),   # 128x256 tiles, three stages
          (4096, 4096, 256, fb.GEMM_TILED),    # 256x256 tiles
          (4096, 4480, 256, fb.GEMM_TILED),    # 256x256 + the 256x192 column split
          (4096, 4096, 1024, fb.GEMM_TILED)]   # 256x256 tiles leaving the main loop at step 2 of 8


@pytest.mark.parametrize("xf,wf", [(fb.E4M3, fb.E4M3), (fb.E4M3, fb.E5M2), (fb.E5M2, fb.E5M2)])
@pytest.mark.parametrize("orient", ["x_small", "x_large"])
def test_mx32_exponents_at_the_ends_of_ue8m0(xf, wf, orient):
    for M, N, K, algo in SHAPES:
        rng = np.random.default_rng(M + N + K + xf * 7 + wf * 3 + (orient == "x_large"))
        lo, hi = (0, 3) if orient == "x_small" else (251, 254)
        # the first quarter of the K blocks foldable: the exact tiled path
        # switches to block-by-block summation midway through K
        nb = (K // 32) // 4
        xq, sx = _crafted(M, K, xf, lo, hi, rng, normal_blocks=nb)
        wq, sw = _crafted(N, K, wf, 254 - hi, 254 - lo, rng, normal_blocks=nb)
        sw[:, :nb] = (254 - sx[0, :nb].astype(np.int64)).astype(np.uint8)   # keep those products ordinary too
        rows = None if M * N <= 1 << 20 else np.random.default_rng(M).choice(M, 48, replace=False)
        for accum in (fb.ACCUM_FP32, fb.ACCUM_NATIVE):
            label = f"mx32 ends {orient} fmt=({xf},{wf}) {M}x{N}x{K} algo={algo} accum={accum}"
            say(label)
            _check(xq, sx, xf, wq, sw, wf, algo, accum, label, rows)


@pytest.mark.parametrize("wf", [fb.E4M3, fb.E5M2])
def test_mx32_quantizer_extremes(wf):
    """Operands from the MX quantizer: X blocks with amax near the fp32 maximum
    (E4M3 e = 120; a code times 2^e exceeds fp32 on its own) against W blocks
    of 1e-30, and X blocks below 448 * 2^-127 (byte 0, nonzero codes) against W
    blocks of 1e30; every product is an ordinary fp32 number."""
    rng = np.random.default_rng(77 + wf)
    for M, N, K, algo in [(16, 256, 512, fb.GEMM_SKINNY), (128, 256, 512, fb.GEMM_TILED)]:
        nb = K // 32
        big = (np.arange(nb) % 2 == 0)                      # alternate block kinds along K
        xs = np.where(np.repeat(big, 32)[None, :], 3.3e38, 1.0e-38).astype(np.float64)
        x = (xs * rng.uniform(0.05, 1.0, (M, K)) * rng.choice([-1.0, 1.0], (M, K))).astype(np.float32)
        x[:, 0] = np.float32(3.4e38)                        # the largest finite-ish value in a big block
        ws = np.where(np.repeat(big, 32)[None, :], 1.0e-30, 1.0e30)
        w = (ws * rng.uniform(0.05, 1.0, (N, K)) * rng.choice([-1.0, 1.0], (N, K))).astype(np.float32)
        xq, sx = quant.quantize(x, MX, fb.E4M3)
        wq, sw = quant.quantize(w, MX, wf)
        assert (sx[:, 0] == 127 + 120).all() and (sx[:, 1] == 0).all()   # the ends the quantizer reaches
        for accum in (fb.ACCUM_FP32, fb.ACCUM_NATIVE):
            label = f"mx32 quantizer extremes wf={wf} {M}x{N}x{K} algo={algo} accum={accum}"
            say(label)
            _check(xq, sx, fb.E4M3, wq, sw, wf, algo, accum, label)


def test_plain_entry_point_through_ctypes():
    """fp8_gemm_blockscaled itself (AUTO kernel, exact accumulation) with raw
    device pointers, for the tiled and the skinny shapes."""
    lib = fb.load_library()
    wl = workloads.CONFIGS["c3_deepseek_block"]
    for M, N, K in [(16, 384, 512), (272, 384, 640)]:
        rng = np.random.default_rng(M * 3 + N)
        x = workloads.draw_x(wl, M, K, rng)
        w = workloads.draw_w(wl, N, K, rng)
        xq, sx = quant.quantize(x, fb.GRAN_TILE_1x128, fb.E4M3)
        wq, sw = quant.quantize(w, fb.GRAN_BLOCK_128x128, fb.E4M3)
        a, sa, b, sb = dev(xq), dev(sx), dev(wq), dev(sw)
        out = torch.empty((M, N), dtype=torch.float32, device="cuda")
        label = f"fp8_gemm_blockscaled via ctypes {M}x{N}x{K}"
        say(label)
        st = lib.fp8_gemm_blockscaled(a.data_ptr(), fb.E4M3, fb.GRAN_TILE_1x128, sa.data_ptr(), b.data_ptr(),
                                      fb.E4M3, fb.GRAN_BLOCK_128x128, sb.data_ptr(), M, N, K, out.data_ptr(),
                                      fb.DT_F32, torch.cuda.current_stream().cuda_stream)
        assert st == 0, fb.fp8_status_string(st)
        torch.cuda.synchronize()
        ref, absb = gemm.gemm_ref(xq, sx, fb.GRAN_TILE_1x128, fb.E4M3, wq, sw, fb.GRAN_BLOCK_128x128, fb.E4M3)
        gemm_check(host(out), fb.DT_F32, ref, absb, label)


def _e4m3(v):
    return int(formats.encode(np.float64(v), formats.E4M3))


@pytest.mark.parametrize("algo", [fb.GEMM_TILED, fb.GEMM_SKINNY])
def test_fp8_matrix_core_group_truncation(algo):
    """Reading G17 on the GPU: eight products in one group, 32 * 32 = 1024
    and 0.9375, 0.5, 0.25, 0.125, 0.0625 (exact sum 1025.875), per-tensor
    scales 1.  The exact path gives the exact sum; the FP8 instruction's own
    accumulation gives a different value whose error exceeds 1e-4 of the sum
    of |products| but stays within 7 * 2^-13 of the largest product."""
    M, N, K = 16, 16, 128
    xq = np.zeros((M, K), np.uint8)
    wq = np.zeros((N, K), np.uint8)
    pairs = [(32.0, 32.0), (1.0, 0.9375), (1.0, 0.5), (1.0, 0.25), (1.0, 0.125), (1.0, 0.0625)]
    for k, (xv, wv) in enumerate(pairs):
        xq[0, k] = _e4m3(xv)
        wq[0, k] = _e4m3(wv)
    exact = sum(xv * wv for xv, wv in pairs)
    one = np.ones(1, np.float32)
    res = {}
    for accum in (fb.ACCUM_FP32, fb.ACCUM_NATIVE):
        say(f"group truncation algo={algo} accum={accum}")
        out = fb.fp8_gemm_blockscaled(dev(xq), fb.E4M3, fb.GRAN_TENSOR, dev(one), dev(wq), fb.E4M3, fb.GRAN_TENSOR,
                                      dev(one), fb.DT_F32, algo=algo, accum=accum)
        torch.cuda.synchronize()
        o = host(out)
        assert (o[1:] == 0).all() and (o[0, 1:] == 0).all()
        res[accum] = float(o[0, 0])
    assert res[fb.ACCUM_FP32] == exact
    err = abs(res[fb.ACCUM_NATIVE] - exact)
    print(f"[case] native accumulation of the crafted group: {res[fb.ACCUM_NATIVE]!r} (exact {exact})", flush=True)
    assert err > 1e-4 * exact, "the FP8 instruction summed the crafted group exactly"
    assert err <= 7 * 2.0 ** -13 * 1024.0
