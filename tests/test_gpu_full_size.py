"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: quantize both operands bit-exactly against the oracle over
the whole tensors, then check the GEMM on sampled output elements against the
oracle's fp64 reference (in the workload's output dtype and in fp32), and the
quantized-output GEMM's codes and scales on sampled rows against the oracle's
quantization of the same kernel's fp32 result."""

import numpy as np
import pytest
import torch

import block_scaled_precision_x128_amd as fb
import workloads
from oracle import gemm
from gpu_helpers import (NATIVE_REL_TOL, assert_codes_equal, assert_scales_equal, dev, full_operands, gemm_check,
                         host, oracle_quantize, say)

pytestmark = pytest.mark.gpu

SAMPLES = 4096


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_full_size_workload(name):
    wl, xs, ws, xq, sx, wq, sw = full_operands(name)
    for operand, store, gran, fmt, wantq, wants in (("x", xs, wl.x_gran, wl.x_fmt, xq, sx),
                                                      ("w", ws, wl.w_gran, wl.w_fmt, wq, sw)):
        rows, cols = store.shape
        say("quantize full size", name, operand, rows, cols)
        q, s = fb.fp8_quantize(dev(store), fmt, gran)
        torch.cuda.synchronize()
        assert_scales_equal(host(s), wants, f"{name}/{operand}")
        assert_codes_equal(host(q), wantq, f"{name}/{operand} codes")
        del q, s
        torch.cuda.empty_cache()

    rng = np.random.default_rng(wl.seed)
    mi = rng.integers(0, wl.M, SAMPLES)
    ni = rng.integers(0, wl.N, SAMPLES)
    um, mi_idx = np.unique(mi, return_inverse=True)
    un, ni_idx = np.unique(ni, return_inverse=True)
    xr = gemm.dequant_rows(xq[um], sx, wl.x_gran, wl.x_fmt, um)
    wr = gemm.dequant_rows(wq[un], sw, wl.w_gran, wl.w_fmt, un)
    ref, absb = gemm.gemm_ref_pairs(xr, wr, mi_idx, ni_idx)

    a, b, sa, sb = dev(xq), dev(wq), dev(sx), dev(sw)
    algos = [fb.GEMM_AUTO] + ([fb.GEMM_TILED] if wl.M <= 64 else [])
    cases = [(algo, fb.ACCUM_FP32, odt, gemm.REL_TOL) for algo in algos for odt in sorted({wl.out_dtype, fb.DT_F32})]
    cases.append((fb.GEMM_AUTO, fb.ACCUM_NATIVE, wl.out_dtype, NATIVE_REL_TOL))
    for algo, accum, odt, rel in cases:
        say("gemm full size", name, "algo", algo, "accum", accum, "odt", odt)
        out = fb.fp8_gemm_blockscaled(a, wl.x_fmt, wl.x_gran, sa, b, wl.w_fmt, wl.w_gran, sb, odt, algo=algo,
                                      accum=accum)
        torch.cuda.synchronize()
        full = out if odt == fb.DT_F32 else out.float()
        assert torch.isfinite(full).all().item()
        got = host(out)[mi, ni]
        worst = gemm_check(got, odt, ref, absb, f"{name} algo={algo} accum={accum} odt={odt}", rel)
        say("worst error / bound", f"{worst:.3g}")
        del out, full

    # The quantized-output GEMM at full size (the launch the benchmark times for
    # the fused epilogue): codes and 1x128 scales of sampled rows, bit for bit,
    # against the oracle's quantization of the same kernel's fp32 rows.
    if wl.N % 128 == 0:
        rows = um[:: max(1, len(um) // 64)]
        for accum in (fb.ACCUM_FP32, fb.ACCUM_NATIVE):
            say("gemm quantized output full size", name, "accum", accum, "rows", len(rows))
            yf = fb.fp8_gemm_blockscaled(a, wl.x_fmt, wl.x_gran, sa, b, wl.w_fmt, wl.w_gran, sb, fb.DT_F32,
                                         algo=fb.GEMM_TILED, accum=accum)
            codes, scales = fb.fp8_gemm_blockscaled_quant(a, wl.x_fmt, wl.x_gran, sa, b, wl.w_fmt, wl.w_gran, sb,
                                                          fb.E4M3, accum=accum)
            torch.cuda.synchronize()
            yh = host(yf)[rows]
            want_q, want_s = oracle_quantize(yh, fb.GRAN_TILE_1x128, fb.E4M3)
            label = f"{name} quantized output accum={accum}"
            assert_scales_equal(host(scales)[rows], want_s, label)
            assert_codes_equal(host(codes)[rows], want_q, label + " codes", yh)
            del yf, codes, scales
    del a, b, sa, sb
    torch.cuda.empty_cache()
