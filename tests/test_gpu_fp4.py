"""GPU parity: FP4 (E2M1) quantize and dequantize with MXFP4 and NVFP4
scaling against the oracle, bit for bit (codes, block scales, tensor scale,
dequantized values; NaN compared as NaN)."""

import numpy as np
import pytest
import torch

import block_scaled_precision_x128_amd as fb
import workloads
from oracle import fp4, quant
from gpu_helpers import assert_codes_equal, dev, host, say

pytestmark = pytest.mark.gpu

KINDS = [fb.FP4_MX, fb.FP4_NV]


def _oracle_quantize(kind, x32):
    if kind == fb.FP4_MX:
        q, s = fp4.quantize_mx(x32)
        return q, s, None
    return fp4.quantize_nv(x32)


def _draw(rng, rows, cols):
    x = rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-6, 6, (rows, 1)))
    x[:, rng.choice(cols, max(1, cols // 64), replace=False)] *= 50        # outlier channels
    x = x.astype(np.float32)
    x[0, :4] = [0.0, -0.0, 1e-30, -1e-30]
    if rows > 2:
        x[2, :] = 0.0                                                       # an all-zero row
    return x


def _check_quantize(kind, dt, x, label):
    store = workloads.f32_to_bf16_bits(x) if dt == fb.DT_BF16 else x
    x32 = workloads.storage_to_f32(store, dt)
    say(label)
    q, bs, ts = fb.fp4_quantize(dev(store), kind)
    torch.cuda.synchronize()
    wq, wbs, wts = _oracle_quantize(kind, x32)
    assert_codes_equal(host(bs), wbs, label + " block scales")
    if kind == fb.FP4_NV:
        assert host(ts).view(np.uint32)[0] == np.float32(wts).view(np.uint32), (label, host(ts), wts)
    assert_codes_equal(host(q), wq, label + " codes", None)
    return q, bs, ts


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dt", [fb.DT_F32, fb.DT_BF16])
@pytest.mark.parametrize("shape", [(1, 128), (33, 256), (96, 1024), (7, 4224)])
def test_fp4_quantize(kind, dt, shape):
    rng = np.random.default_rng(500 + 10 * kind + dt + shape[1])
    _check_quantize(kind, dt, _draw(rng, *shape), f"fp4 quantize kind={kind} dt={dt} shape={shape}")


def test_fp4_mx_ties_and_saturation():
    """Every E2M1 rounding midpoint, times the block's power of two, in blocks
    whose largest element fixes the exponent."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.2500001, 5.0000001, 1.0, 3.0, 0.5])
    rows, cols = 8, 128
    x = np.zeros((rows, cols), np.float64)
    for r in range(rows):
        for b in range(cols // 32):
            e = (r * 7 + b * 3) % 40 - 20
            v = np.concatenate([[6.0], mids, -mids, [0.1, -0.1, 5.9, -5.9, 0.74, 0.76, 2.4, 2.6, 4.9]])[:32]
            x[r, 32 * b:32 * b + 32] = v * 2.0 ** e
    _check_quantize(fb.FP4_MX, fb.DT_F32, x.astype(np.float32), "fp4 MX ties")


def test_fp4_nv_extremes():
    """A block whose microscale rounds to zero (signed-zero codes), a block at
    the tensor amax (microscale 448), subnormal inputs, and an empty tensor."""
    x = np.zeros((4, 128), np.float32)
    x[0, 0] = 3e38
    x[1, :16] = 1e-30
    x[1, 16:32] = -2.0 ** -140
    x[2, :] = np.linspace(-3e36, 3e36, 128, dtype=np.float32)
    _check_quantize(fb.FP4_NV, fb.DT_F32, x, "fp4 NV extremes")
    say("fp4 NV empty")
    q, bs, ts = fb.fp4_quantize(torch.zeros((0, 128), device="cuda"), fb.FP4_NV)
    torch.cuda.synchronize()
    assert host(ts)[0] == 1.0


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("out_dt", [fb.DT_F32, fb.DT_BF16])
def test_fp4_dequantize(kind, out_dt):
    rng = np.random.default_rng(600 + kind + 2 * out_dt)
    rows, cols = 40, 512
    q = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    if kind == fb.FP4_MX:
        bs = rng.integers(90, 170, (rows, cols // 32)).astype(np.uint8)
        bs[0, 0], bs[1, 1], bs[2, 2] = 255, 0, 254
        ts = None
        want = fp4.dequantize_mx(q, bs)
    else:
        bs = rng.integers(0, 256, (rows, cols // 16)).astype(np.uint8)   # includes the E4M3 NaN codes
        ts = np.array([0.0123], np.float32)
        want = fp4.dequantize_nv(q, bs, ts[0])
    label = f"fp4 dequantize kind={kind} out={out_dt}"
    say(label)
    y = fb.fp4_dequantize(dev(q), dev(bs), None if ts is None else dev(ts), kind, out_dt)
    torch.cuda.synchronize()
    got = host(y)
    if out_dt == fb.DT_F32:
        nan_g, nan_w = np.isnan(got), np.isnan(want)
        assert np.array_equal(nan_g, nan_w), label
        assert_codes_equal(np.where(nan_g, 0, got.view(np.uint32)), np.where(nan_w, 0, want.view(np.uint32)), label)
    else:
        wb = quant.to_bf16_bits(want)
        nan_g, nan_w = (got & 0x7FFF) > 0x7F80, (wb & 0x7FFF) > 0x7F80
        assert np.array_equal(nan_g, nan_w), label
        assert_codes_equal(np.where(nan_g, 0, got), np.where(nan_w, 0, wb), label)


@pytest.mark.parametrize("kind", KINDS)
def test_fp4_round_trip_full_width(kind):
    """Quantize on the GPU, dequantize on the GPU, against the oracle's round
    trip, at a 7168-wide bf16 operand (the DeepSeek hidden size)."""
    rng = np.random.default_rng(700 + kind)
    x = workloads.f32_to_bf16_bits(_draw(rng, 64, 7168))
    q, bs, ts = _check_quantize(kind, fb.DT_BF16, workloads.bf16_bits_to_f32(x), f"fp4 full width kind={kind}")
    y = fb.fp4_dequantize(q, bs, ts, kind, fb.DT_F32)
    torch.cuda.synchronize()
    wq, wbs, wts = _oracle_quantize(kind, workloads.bf16_bits_to_f32(x))
    want = fp4.dequantize_mx(wq, wbs) if kind == fb.FP4_MX else fp4.dequantize_nv(wq, wbs, wts)
    assert_codes_equal(host(y).view(np.uint32), want.view(np.uint32), "fp4 round trip")


@pytest.mark.parametrize("dt", [fb.DT_F32, fb.DT_BF16])
def test_fp4_mx_every_bf16_value(dt):
    """The E2M1 cast on every bf16 value of magnitude at most 6 (both signs,
    zeros and bf16 subnormals included): each sits in an MX block whose first
    element is 6, so the block exponent is 0 and the codes are the unscaled
    cast.  The fp32 input also carries fp32 subnormals, which must round to
    signed zeros."""
    bits = np.arange(0, 0x10000, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 6.0)]
    if dt == fb.DT_F32:
        vals = np.concatenate([vals, np.array([1e-40, -1e-40, 1.4e-45, -1.4e-45, -3e-39], np.float32)])
    per_block = 31
    nblk = -(-vals.size // per_block)
    nblk += (-nblk) % 4                       # rows of 128 elements (4 blocks)
    x = np.zeros((nblk, 32), np.float32)
    x[:, 0] = 6.0
    flat = np.zeros(nblk * per_block, np.float32)
    flat[:vals.size] = vals
    x[:, 1:] = flat.reshape(nblk, per_block)
    _check_quantize(fb.FP4_MX, dt, x.reshape(nblk // 4, 128), f"fp4 MX every bf16 value dt={dt}")


@pytest.mark.parametrize("pos", ["last", "fourth_slot"])
def test_fp4_nv_quantize_many_trips(pos):
    """NVFP4 at 4096 x 4608 bf16 (18.9 M elements): both passes cap their
    grids, so every thread loops over several chunks a grid stride apart.
    The tensor's largest magnitude sits in its last element or in a chunk
    reached only on a later trip, so a skipped chunk changes the tensor scale
    and every code."""
    rng = np.random.default_rng(880 + len(pos))
    rows, cols = 4096, 4608
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    flat = x.reshape(-1)
    stride = 2048 * 256                      # chunks of 8 elements per grid stride
    at = flat.size - 1 if pos == "last" else 8 * (3 * stride + 5) + 3
    flat[at] = -4096.0
    _check_quantize(fb.FP4_NV, fb.DT_BF16, x, f"fp4 NV many trips pos={pos}")
