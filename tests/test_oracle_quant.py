"""Pins for the oracle's scale rules, groups, quantize and dequantize (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from oracle import formats, quant
from oracle.formats import E4M3, E5M2


def rn32_exact(q: Fraction) -> np.float32:
    """Round an exact rational to fp32 (nearest, ties to even) by comparing
    exact distances to the neighbouring fp32 numbers."""
    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        key = (abs(Fraction(float(c)) - q), int(np.array(c).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def _amax_samples(rng):
    m = rng.integers(0, 2 ** 23, 3000)
    e = rng.integers(-100, 100, 3000)
    a = np.ldexp(1.0 + m / 2.0 ** 23, e)
    special = np.array([448.0, 57344.0, 1.0, 2.0 ** -126, 1e-38, 3.0e38, 448 * 1.75, 0.0021])
    return np.concatenate([a, special]).astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("f", [E4M3, E5M2])
def test_fp32_scale_is_correctly_rounded(f):
    rng = np.random.default_rng(1)
    amax = _amax_samples(rng)
    s = quant.fp32_scale(amax, f)
    vmax = Fraction(f.vmax)
    for a, got in zip(amax, s):
        want = rn32_exact(Fraction(float(a)) / vmax)
        if want == 0:
            want = np.float32(1.0)
        assert np.float32(got) == want, (a, got, want)


def test_scaled_quotient_is_correctly_rounded():
    """The element step RN32(x / s) against exact rational rounding, including
    quotients that land on FP8 rounding midpoints."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal(4000).astype(np.float32).astype(np.float64)
    s = np.float32(rng.uniform(1e-3, 1.0))
    mids = np.array([232.0, 248.0, 17.0, 19.0, 2.0 ** -10, 464.0])
    x = np.concatenate([x, (mids * np.float64(s)).astype(np.float32).astype(np.float64)])
    q = (x / np.float64(s)).astype(np.float32)
    for xi, qi in zip(x, q):
        assert qi == rn32_exact(Fraction(float(xi)) / Fraction(float(s)))


@pytest.mark.parametrize("f", [E4M3, E5M2])
def test_mx_exponent_bruteforce(f):
    rng = np.random.default_rng(3)
    amax = _amax_samples(rng)
    e = quant.mx_exponent(amax, f)
    vmax = Fraction(f.vmax)
    for a, got in zip(amax, e):
        if a == 0:
            assert got == -127
            continue
        fa = Fraction(float(a))
        k = -300
        while not fa <= vmax * Fraction(2) ** k:
            k += 1
        assert got == max(-127, min(127, k)), (a, got, k)


@pytest.mark.parametrize("gran", [quant.TENSOR, quant.ROW, quant.TILE_1x128, quant.BLOCK_128x128, quant.MX32])
def test_group_layout(gran):
    """Each group gets a distinct amax; the scale array must put it at the
    documented index (catches transposed or mis-strided layouts)."""
    rows, cols = 256, 512
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :]
    if gran == quant.ROW:
        gid = r + 0 * c
    elif gran == quant.TILE_1x128:
        gid = r * (cols // 128) + c // 128
    elif gran == quant.BLOCK_128x128:
        gid = (r // 128) * (cols // 128) + c // 128
    elif gran == quant.MX32:
        gid = r * (cols // 32) + c // 32
    else:
        gid = 0 * r + 0 * c
    # amax of group g is 2^(g mod 40 - 20) * 1.5, placed at one element per group
    x = np.full((rows, cols), 0.0, dtype=np.float32)
    amax_g = np.ldexp(1.5, (gid % 40) - 20).astype(np.float32)
    first = np.zeros_like(gid, dtype=bool)
    _, idx = np.unique(gid.reshape(-1), return_index=True)
    first.reshape(-1)[idx] = True
    x[first] = amax_g[first]
    x[~first] = amax_g[~first] * np.float32(0.25)
    codes, scales = quant.quantize(x, gran, E4M3)
    assert scales.shape == quant.scale_shape(gran, rows, cols)
    if gran == quant.MX32:
        e = scales.astype(np.int64) - 127
        # smallest e with 1.5*2^k <= 448*2^e: 448 = 1.75*2^8 -> e = k - 8
        want = (np.arange(scales.size) % 40 - 20) - 8
        assert np.array_equal(e.reshape(-1), want)
    else:
        want = (np.ldexp(1.5, (np.arange(scales.size) % 40) - 20) / 448.0).astype(np.float32)
        assert np.array_equal(scales.reshape(-1), want)


@pytest.mark.parametrize("f", [E4M3, E5M2])
@pytest.mark.parametrize("gran", [quant.TENSOR, quant.ROW, quant.TILE_1x128, quant.BLOCK_128x128])
def test_fp32_group_max_hits_vmax(f, gran):
    """Every nonzero group has |amax / s| rounding to Vmax: its largest code is
    the Vmax code, and no larger magnitude appears."""
    wl = workloads.CONFIGS["c3_deepseek_block"]
    x = workloads.draw_x(wl, 256, 512, np.random.default_rng(9))
    codes, s = quant.quantize(x, gran, f)
    mag = (codes & 0x7F).astype(np.int64)
    vcode = formats.vmax_code(f)
    assert mag.max() == vcode
    if gran == quant.TILE_1x128:
        assert np.all(mag.reshape(256, 4, 128).max(axis=2) == vcode)
    if gran == quant.ROW:
        assert np.all(mag.max(axis=1) == vcode)


@pytest.mark.parametrize("f", [E4M3, E5M2])
def test_mx_no_saturation_and_block_max_range(f):
    wl = workloads.CONFIGS["c5_mxfp8_mix"]
    x = workloads.draw_w(wl, 64, 256, np.random.default_rng(4))
    codes, e = quant.quantize(x, quant.MX32, f)
    vals = np.abs(formats.decode(codes, f)).reshape(64, 8, 32)
    bmax = vals.max(axis=2)
    assert np.all(bmax <= f.vmax) and np.all(bmax >= f.vmax / 2)
    # exact: decoded * 2^e reproduces x within FP8's relative rounding (normal range)
    xh = quant.dequantize(codes, e, quant.MX32, f).astype(np.float64)
    big = np.abs(x) >= np.repeat(np.ldexp(2.0 ** f.emin, e.astype(np.int64) - 127), 32, axis=1)
    rel = np.abs(xh - x)[big] / np.abs(x)[big]
    assert rel.max() <= 2.0 ** -(f.mbits + 1)


def test_zero_groups():
    x = np.zeros((2, 128), np.float32)
    x[1, 5] = -0.0
    for gran in (quant.TENSOR, quant.ROW, quant.TILE_1x128):
        codes, s = quant.quantize(x, gran, E4M3)
        assert np.all(s == 1.0)
        assert np.all((codes & 0x7F) == 0)
    codes, e = quant.quantize(x, quant.MX32, E4M3)
    assert np.all(e == 0) and np.all(codes & 0x7F == 0)   # byte 0 == e of -127


def test_dequantize_values():
    codes = np.array([[0x38, 0x40, 0xB8, 0x7E]], dtype=np.uint8)   # 1, 2, -1, 448
    s = np.array([0.5], np.float32)
    y = quant.dequantize(codes, s, quant.TENSOR, E4M3)
    assert y.tolist() == [[0.5, 1.0, -0.5, 224.0]]
    e = np.full((1, 4), 127 + 3, np.uint8)
    codes = np.tile(codes, (1, 32))
    y = quant.dequantize(codes, e, quant.MX32, E4M3)
    assert y[0, :4].tolist() == [8.0, 16.0, -8.0, 3584.0]
    e255 = np.full((1, 4), 255, np.uint8)
    assert np.isnan(quant.dequantize(codes, e255, quant.MX32, E4M3)).all()


def test_dequantize_round_is_single_fp32_rounding():
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 256, (16, 128), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10
    s = rng.uniform(1e-3, 10, (16, 1)).astype(np.float32)
    y = quant.dequantize(codes, s.reshape(-1), quant.ROW, E4M3)
    for i in range(16):
        for j in range(0, 128, 7):
            want = rn32_exact(Fraction(formats.decode_code(int(codes[i, j]), E4M3)) * Fraction(float(s[i, 0])))
            assert y[i, j] == want


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(8)
    bits = rng.integers(0, 2 ** 32, 300000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    v = np.concatenate([v, np.array([3.4e38, -3.4e38, 0.0, -0.0, 1e-45], np.float32)])
    ours = quant.to_bf16_bits(v)
    theirs = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_shape_rules():
    with pytest.raises(ValueError):
        quant.quantize(np.zeros((4, 100), np.float32), quant.ROW, E4M3)
    with pytest.raises(ValueError):
        quant.quantize(np.zeros((100, 128), np.float32), quant.BLOCK_128x128, E4M3)


def test_input_generator_is_deterministic():
    wl = workloads.CONFIGS["c2_per_token_channel"]
    a = workloads.make_inputs(wl, 64, 32, 512)
    b = workloads.make_inputs(wl, 64, 32, 512)
    assert all(np.array_equal(p, q) for p, q in zip(a, b))
    assert a[0].dtype == np.uint16 and a[0].shape == (64, 512) and a[1].shape == (32, 512)
    x = workloads.storage_to_f32(a[0], wl.in_dtype)
    col_amax = np.abs(x).max(axis=0)
    assert (col_amax > 15).sum() == wl.n_outliers(512) == 5
    # storage cast equals torch's bf16 rounding
    xf = workloads.draw_x(wl, 64, 512, np.random.default_rng(wl.seed))
    tb = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(workloads.f32_to_bf16_bits(xf), tb)


# ---- delayed scaling ("FP8 Mixed-Precision Serving", delayed scaling) --------

def test_delayed_scale_closed_forms():
    E4M3, E5M2 = 0, 1
    assert quant.delayed_scale(np.zeros(4, np.float32), 0, E4M3) == np.float32(1.0)   # empty history
    assert quant.delayed_scale(np.array([1.0, 448.0, 3.0], np.float32), 0, E4M3) == np.float32(1.0)
    assert quant.delayed_scale(np.array([1.0, 448.0, 3.0], np.float32), 2, E4M3) == np.float32(4.0)
    assert quant.delayed_scale(np.array([57344.0], np.float32), 0, E5M2) == np.float32(1.0)
    assert quant.delayed_scale(np.array([np.nan, 896.0], np.float32), 0, E4M3) == np.float32(2.0)


def test_delayed_scale_is_correctly_rounded():
    """Against exact rational arithmetic: s = RN32(2^m max(H) / Vmax)."""
    from fractions import Fraction
    rng = np.random.default_rng(11)
    for _ in range(500):
        h = (rng.random(8) * 10.0 ** rng.integers(-30, 30)).astype(np.float32)
        m = int(rng.integers(0, 8))
        exact = Fraction(float(h.max())) * 2 ** m / 448
        s = quant.delayed_scale(h, m, 0)
        lo, hi = np.nextafter(s, np.float32(0)), np.nextafter(s, np.float32(np.inf))
        # s is the nearest fp32 to the exact quotient
        assert abs(Fraction(float(s)) - exact) <= abs(Fraction(float(lo)) - exact)
        assert abs(Fraction(float(s)) - exact) <= abs(Fraction(float(hi)) - exact)


def test_quantize_delayed_saturates_and_updates_history():
    """A spike larger than the history allows clips to +-Vmax (the overflow
    risk the page names); the history entry then holds the spike's amax."""
    h = np.array([2.0, 1.0, 0.0], np.float32)
    x = np.array([[0.5, -1.0, 2.0, 50.0, -50.0, 0.0, 1.5, -2.0]], np.float32)
    codes, s, h2 = quant.quantize_delayed(x, h, 2, 0, 0)
    assert s == np.float32(2.0 / 448.0)
    assert codes[0, 3] == 0x7E and codes[0, 4] == 0xFE          # +-448 after saturation
    assert codes[0, 2] == 0x7E                                    # 2.0 / s = 448 exactly
    assert h2.tolist() == [2.0, 1.0, 50.0] and h.tolist() == [2.0, 1.0, 0.0]
    # with the current scale the same tensor would not clip
    xp = np.zeros((1, 128), np.float32)
    xp[:, :8] = x
    q_cur, s_cur = quant.quantize(xp, quant.TENSOR, 0)
    assert s_cur[0] == np.float32(50.0 / 448.0) and q_cur[0, 3] == 0x7E


def test_delayed_equals_current_scaling_when_history_holds_the_amax():
    """With max(H) = amax(x) and no margin the delayed codes are the per-tensor ones."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    h = np.array([np.abs(x).max(), 0.5], np.float32)
    codes, s, _ = quant.quantize_delayed(x, h, 1, 0, 0)
    q_cur, s_cur = quant.quantize(x, quant.TENSOR, 0)
    assert s == s_cur[0] and np.array_equal(codes, q_cur)
