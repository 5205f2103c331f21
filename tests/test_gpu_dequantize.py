"""GPU parity: dequantize, bit-exact against the oracle (NaN compared as NaN)."""

import numpy as np
import pytest
import torch

import block_scaled_precision_x128_amd as fb
from oracle import quant
from gpu_helpers import assert_codes_equal, dev, host, say

pytestmark = pytest.mark.gpu


def _scales(gran, rows, cols, rng):
    shp = fb.scale_shape(gran, rows, cols)
    if gran == fb.GRAN_MX32:
        e = rng.integers(0, 256, shp).astype(np.uint8)   # includes 255 (NaN) and the extremes
        return e
    s = np.exp(rng.uniform(-60, 60, shp)).astype(np.float32)
    flat = s.reshape(-1)
    if flat.size >= 3:
        flat[:3] = [1e-40, 3e38, 1.0]     # subnormal scale, overflow to Inf, identity
    return s


@pytest.mark.parametrize("gran", [fb.GRAN_TENSOR, fb.GRAN_ROW, fb.GRAN_TILE_1x128, fb.GRAN_BLOCK_128x128,
                                  fb.GRAN_MX32])
@pytest.mark.parametrize("fmt", [fb.E4M3, fb.E5M2])
@pytest.mark.parametrize("odt", [fb.DT_F32, fb.DT_BF16])
def test_dequantize_all_codes(gran, fmt, odt):
    say("dequantize", gran, fmt, odt)
    rng = np.random.default_rng(gran * 10 + fmt)
    rows, cols = 256, 512
    codes = np.tile(np.arange(256, dtype=np.uint8), rows * cols // 256).reshape(rows, cols)
    rng.shuffle(codes, axis=1)
    s = _scales(gran, rows, cols, rng)
    y = fb.fp8_dequantize(dev(codes), dev(s), fmt, gran, odt)
    torch.cuda.synchronize()
    want = quant.dequantize(codes, s, gran, fmt)
    got = host(y)
    if odt == fb.DT_F32:
        nan_g, nan_w = np.isnan(got), np.isnan(want)
        assert np.array_equal(nan_g, nan_w)
        assert_codes_equal(np.where(nan_g, 0, got.view(np.uint32)), np.where(nan_w, 0, want.view(np.uint32)),
                           "dequant f32")
    else:
        wb = quant.to_bf16_bits(want)
        nan_g = (got & 0x7FFF) > 0x7F80
        nan_w = (wb & 0x7FFF) > 0x7F80
        assert np.array_equal(nan_g, nan_w)
        assert_codes_equal(np.where(nan_g, 0, got), np.where(nan_w, 0, wb), "dequant bf16")
