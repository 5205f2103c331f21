"""GPU parity: delayed scaling over a sequence of iterations.

Each iteration quantizes a new tensor with the scale taken from the amax
history of the earlier ones and then records its own amax; the codes, the
scale and the whole history must match the oracle bit for bit at every step,
including a step whose spike exceeds what the history allows (saturation)."""

import numpy as np
import pytest
import torch

import block_scaled_precision_x128_amd as fb
import workloads
from oracle import quant
from gpu_helpers import assert_codes_equal, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", [fb.E4M3, fb.E5M2])
@pytest.mark.parametrize("dt", [fb.DT_F32, fb.DT_BF16])
@pytest.mark.parametrize("margin", [0, 2])
def test_delayed_scaling_sequence(fmt, dt, margin):
    rng = np.random.default_rng(100 + fmt + 2 * dt + margin)
    wl = workloads.CONFIGS["c2_per_token_channel"]
    hlen = 4
    hist_o = np.zeros(hlen, np.float32)
    hist_d = torch.zeros(hlen, dtype=torch.float32, device="cuda")
    for it in range(7):
        rows, cols = (96, 640) if it % 2 else (33, 1024)
        x = workloads.draw_x(wl, rows, cols, rng) * np.float32(1.0 + it)
        if it == 4:
            x[5, 7] = np.float32(4000.0)          # a spike the history does not cover
        x_store = workloads.f32_to_bf16_bits(x) if dt == fb.DT_BF16 else x
        x32 = workloads.storage_to_f32(x_store, dt)
        pos = it % hlen
        label = f"delayed fmt={fmt} dt={dt} margin={margin} iteration={it}"
        say(label)
        q, s = fb.fp8_quantize_delayed(dev(x_store), fmt, hist_d, pos, margin)
        torch.cuda.synchronize()
        want_q, want_s, hist_o = quant.quantize_delayed(x32, hist_o, pos, margin, fmt)
        assert host(s).view(np.uint32)[0] == np.float32(want_s).view(np.uint32), (label, host(s), want_s)
        assert_codes_equal(host(q), want_q, label + " codes", x32)
        assert np.array_equal(host(hist_d).view(np.uint32), hist_o.view(np.uint32)), (label, host(hist_d), hist_o)


@pytest.mark.parametrize("fmt", [fb.E4M3, fb.E5M2])
def test_delayed_scale_far_from_the_data(fmt):
    """A history far below the data (quotients beyond the fp32 range: codes
    saturate, E5M2 never gives Inf) and a history whose scale overflows fp32
    (scale +Inf: codes are signed zeros)."""
    cases = [("tiny history", np.array([1e-30, 0.0], np.float32), 0),
             ("scale overflows", np.array([3e38, 1.0], np.float32), 31)]
    rng = np.random.default_rng(55 + fmt)
    for name, hist, margin in cases:
        x = (rng.standard_normal((8, 128)) * 10).astype(np.float32)
        x[0, :4] = [1e30, -1e30, 0.0, -0.0]
        label = f"delayed extreme fmt={fmt} {name}"
        say(label)
        hist_d = dev(hist.copy())
        q, s = fb.fp8_quantize_delayed(dev(x), fmt, hist_d, 1, margin)
        torch.cuda.synchronize()
        want_q, want_s, want_h = quant.quantize_delayed(x, hist, 1, margin, fmt)
        assert host(s).view(np.uint32)[0] == np.float32(want_s).view(np.uint32), (label, host(s), want_s)
        assert_codes_equal(host(q), want_q, label + " codes", x)
        assert np.array_equal(host(hist_d).view(np.uint32), want_h.view(np.uint32)), label


@pytest.mark.parametrize("hlen", [1000, 4096, 4097, 10000])
def test_delayed_long_history(hlen):
    """Histories of up to 4096 entries are scanned by every wave of the encode
    kernel; longer ones by a separate one-workgroup kernel.  Both reductions
    keep several loads in flight per thread, with a tail for lengths that are
    not a multiple of that stride: the maximum sits in the tail, NaN entries
    are skipped, and the scale, codes and history must match the oracle bit
    for bit."""
    rng = np.random.default_rng(300 + hlen)
    hist = rng.uniform(0.0, 5.0, hlen).astype(np.float32)
    hist[rng.choice(hlen, 7, replace=False)] = np.float32(np.nan)
    hist[hlen - 1] = np.float32(37.5)             # the maximum, in the last (tail) entry
    pos = hlen // 3
    fmt = fb.E4M3
    x = (rng.standard_normal((64, 384)) * 4).astype(np.float32)
    label = f"delayed long history len={hlen}"
    say(label)
    hist_d = dev(hist.copy())
    q, s = fb.fp8_quantize_delayed(dev(x), fmt, hist_d, pos, 1)
    torch.cuda.synchronize()
    want_q, want_s, want_h = quant.quantize_delayed(x, hist, pos, 1, fmt)
    assert host(s).view(np.uint32)[0] == np.float32(want_s).view(np.uint32), (label, host(s), want_s)
    assert_codes_equal(host(q), want_q, label + " codes", x)
    got_h = host(hist_d)
    assert np.array_equal(np.isnan(got_h), np.isnan(want_h)), label
    ok = ~np.isnan(want_h)
    assert np.array_equal(got_h[ok].view(np.uint32), want_h[ok].view(np.uint32)), label
