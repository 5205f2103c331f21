"""GPU parity: unscaled cast and quantize, bit-exact against the oracle."""

import numpy as np
import pytest
import torch

import block_scaled_precision_x128_amd as fb
import workloads
from oracle import formats, quant
from gpu_helpers import assert_codes_equal, assert_scales_equal, dev, f32_of_store, host, oracle_quantize, say

pytestmark = pytest.mark.gpu

FMTS = [fb.E4M3, fb.E5M2]
GRANS = [fb.GRAN_TENSOR, fb.GRAN_ROW, fb.GRAN_TILE_1x128, fb.GRAN_BLOCK_128x128, fb.GRAN_MX32]


@pytest.mark.parametrize("fmt", FMTS)
def test_cast_exhaustive_bf16(fmt):
    say("cast bf16 exhaustive", fmt)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    q = host(fb.fp8_cast(dev(bits), fmt))
    want = formats.encode(workloads.bf16_bits_to_f32(bits).astype(np.float64), fmt)
    assert_codes_equal(q, want, f"cast bf16 fmt={fmt}", workloads.bf16_bits_to_f32(bits))


@pytest.mark.parametrize("fmt", FMTS)
def test_cast_fp32_specials_ties_random(fmt):
    say("cast fp32", fmt)
    rng = np.random.default_rng(100 + fmt)
    t = formats.decode_table(fmt)
    pos = np.sort(t[:128][np.isfinite(t[:128])])
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    vals = np.concatenate([
        mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf)),
        pos.astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, np.nan, -np.nan, 3.4e38, -3.4e38, 1e-45, -1e-45,
                  1e-38, 448.0, 464.0, 465.0, 480.0, 57344.0, 61440.0, 61441.0, 65536.0], np.float32),
        rng.integers(0, 2 ** 32, 1 << 20, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ]).astype(np.float32)
    vals = np.concatenate([vals, -vals])
    vals = vals[: len(vals) // 8 * 8]
    q = host(fb.fp8_cast(dev(vals), fmt))
    want = formats.encode(vals.astype(np.float64), fmt)
    assert_codes_equal(q, want, f"cast fp32 fmt={fmt}", vals)


def _adversarial_rows(rows, cols, fmt, rng):
    """Each 128-column tile: one element sets amax, the others are chosen so
    that x / s lands on or next to FP8 rounding midpoints (double-rounding and
    tie cases of the correctly rounded division)."""
    t = formats.decode_table(fmt)
    pos = np.sort(t[:128][np.isfinite(t[:128])])
    mids = (pos[:-1] + pos[1:]) / 2
    vmax = pos[-1]
    x = np.empty((rows, cols), np.float32)
    for r in range(rows):
        for kb in range(cols // 128):
            amax = np.float32(np.exp(rng.uniform(-20, 20)))
            s = np.float32(np.float64(amax) / vmax)
            m = rng.choice(mids[mids < vmax], 127)
            base = (m * np.float64(s)).astype(np.float32)
            jitter = rng.integers(-2, 3, 127)
            v = (base.view(np.int32) + jitter).astype(np.int32).view(np.float32)
            v = np.where(np.abs(v) <= amax, v, base)
            sign = np.where(rng.integers(0, 2, 127) == 1, 1, -1).astype(np.float32)
            tile = np.concatenate([[amax], v * sign]).astype(np.float32)
            x[r, kb * 128:(kb + 1) * 128] = tile
    return x


def _run_quant(x_store, gran, fmt, label):
    xd = dev(x_store)
    q, s = fb.fp8_quantize(xd, fmt, gran)
    torch.cuda.synchronize()
    wq, ws = oracle_quantize(x_store, gran, fmt)
    assert_scales_equal(host(s), ws, label)
    assert_codes_equal(host(q), wq, label + " codes", f32_of_store(x_store))


@pytest.mark.parametrize("gran", GRANS)
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dt", [fb.DT_F32, fb.DT_BF16])
def test_quantize_ragged_shapes(gran, fmt, dt):
    wl = workloads.CONFIGS["c3_deepseek_block"]
    for rows, cols in [(1, 128), (3, 384), (256, 640), (384, 1152)]:
        if gran == fb.GRAN_BLOCK_128x128 and rows % 128:
            continue
        say("quantize", gran, fmt, dt, rows, cols)
        x = workloads.draw_x(wl, rows, cols, np.random.default_rng(rows * 7 + cols))
        x_store = workloads.f32_to_bf16_bits(x) if dt == fb.DT_BF16 else x
        _run_quant(x_store, gran, fmt, f"g={gran} f={fmt} dt={dt} {rows}x{cols}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dt", [fb.DT_F32, fb.DT_BF16])
def test_quantize_row_lengths(fmt, dt):
    """Per-row scales over every row-length class of the row kernels (one
    workgroup per row holding 2, 4 or 8 chunks of 8 elements per thread, and
    the two-pass kernel for longer rows)."""
    wl = workloads.CONFIGS["c2_per_token_channel"]
    for cols in (2560, 4096, 6272, 8192, 12288, 20480):
        rows = 5
        say("quantize row lengths", fmt, dt, rows, cols)
        x = workloads.draw_x(wl, rows, cols, np.random.default_rng(cols + fmt))
        x_store = workloads.f32_to_bf16_bits(x) if dt == fb.DT_BF16 else x
        _run_quant(x_store, fb.GRAN_ROW, fmt, f"row lengths f={fmt} dt={dt} {rows}x{cols}")


@pytest.mark.parametrize("gran", GRANS)
@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_adversarial_quotients(gran, fmt):
    say("quantize adversarial", gran, fmt)
    x = _adversarial_rows(128, 256, fmt, np.random.default_rng(5 + gran + 10 * fmt))
    _run_quant(x, gran, fmt, f"adversarial g={gran} f={fmt}")


@pytest.mark.parametrize("gran", GRANS)
def test_quantize_degenerate_groups(gran):
    """All-zero groups, -0, tiny amax (fp32 subnormal scales), huge values."""
    say("quantize degenerate", gran)
    rows, cols = 128, 512
    x = np.zeros((rows, cols), np.float32)
    x[1, :] = -0.0
    rng = np.random.default_rng(77)
    x[2, :] = rng.standard_normal(cols).astype(np.float32) * np.float32(1e-38)
    x[3, :] = rng.standard_normal(cols).astype(np.float32) * np.float32(1e-42)
    x[4, :] = rng.standard_normal(cols).astype(np.float32) * np.float32(1e37)
    x[5, :128] = 3.4e38
    x[5, 128:] = -3.4e38
    x[6, ::2] = 1e-45
    x[7, :] = rng.standard_normal(cols).astype(np.float32)
    x[7, 5] = -0.0
    for fmt in FMTS:
        _run_quant(x, gran, fmt, f"degenerate g={gran} f={fmt}")


def test_quantize_empty_tensor_scale():
    say("quantize empty")
    x = torch.empty((0, 128), dtype=torch.float32, device="cuda")
    q, s = fb.fp8_quantize(x, fb.E4M3, fb.GRAN_TENSOR)
    torch.cuda.synchronize()
    assert host(s).tolist() == [1.0]


def test_quantize_deterministic():
    say("quantize repeat")
    wl = workloads.CONFIGS["c3_deepseek_block"]
    x = dev(workloads.f32_to_bf16_bits(workloads.draw_x(wl, 512, 2048, np.random.default_rng(1))))
    outs = [fb.fp8_quantize(x, fb.E4M3, fb.GRAN_TILE_1x128) for _ in range(3)]
    torch.cuda.synchronize()
    for q, s in outs[1:]:
        assert torch.equal(q, outs[0][0]) and torch.equal(s, outs[0][1])
