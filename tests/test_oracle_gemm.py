"""Pins for the oracle's block-scaled GEMM and its tolerance (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import formats, gemm, quant
from oracle.formats import E4M3, E5M2


def _rand_codes(rng, shape, f):
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    t = formats.decode_table(f)
    bad = ~np.isfinite(t[c])
    c[bad] = 0x30
    return c


def _scales(rng, gran, rows, cols):
    shp = quant.scale_shape(gran, rows, cols)
    if gran == quant.MX32:
        return rng.integers(110, 140, shp).astype(np.uint8)
    return rng.uniform(1e-3, 4.0, shp).astype(np.float32)


@pytest.mark.parametrize("xg,wg,xf,wf", [
    (quant.TENSOR, quant.TENSOR, E4M3, E4M3),
    (quant.ROW, quant.ROW, E4M3, E4M3),
    (quant.TILE_1x128, quant.BLOCK_128x128, E4M3, E4M3),
    (quant.MX32, quant.MX32, E4M3, E5M2),
])
def test_fraction_bruteforce_tiny(xg, wg, xf, wf):
    rng = np.random.default_rng(21)
    M, N, K = 3, 128, 256
    xq = _rand_codes(rng, (M, K), xf)
    wq = _rand_codes(rng, (N, K), wf)
    sx = _scales(rng, xg, M, K) if xg != quant.BLOCK_128x128 else None
    sw = _scales(rng, wg, N, K)
    ref, absb = gemm.gemm_ref(xq, sx, xg, xf, wq, sw, wg, wf)
    tx = formats.decode_table(xf)
    tw = formats.decode_table(wf)

    def scale(s, g, r, k):
        if g == quant.TENSOR:
            return Fraction(float(s.reshape(-1)[0]))
        if g == quant.ROW:
            return Fraction(float(s[r]))
        if g == quant.TILE_1x128:
            return Fraction(float(s[r, k // 128]))
        if g == quant.BLOCK_128x128:
            return Fraction(float(s[r // 128, k // 128]))
        return Fraction(2) ** (int(s[r, k // 32]) - 127)

    for m in range(M):
        for n in (0, 5, 77, 127):
            exact = sum(Fraction(tx[xq[m, k]]) * scale(sx, xg, m, k) *
                        Fraction(tw[wq[n, k]]) * scale(sw, wg, n, k) for k in range(K))
            assert abs(Fraction(float(ref[m, n])) - exact) <= Fraction(2) ** -45 * Fraction(float(absb[m, n]))


def test_integer_codes_give_exact_integer_matmul():
    """Codes of integers in [-16, 16] (all exact in E4M3) with unit scales make
    the GEMM an integer matmul."""
    rng = np.random.default_rng(22)
    M, N, K = 16, 32, 256
    xi = rng.integers(-16, 17, (M, K))
    wi = rng.integers(-16, 17, (N, K))
    xq = formats.encode(xi.astype(np.float64), E4M3)
    wq = formats.encode(wi.astype(np.float64), E4M3)
    one = np.ones(1, np.float32)
    ref, _ = gemm.gemm_ref(xq, one, quant.TENSOR, E4M3, wq, one, quant.TENSOR, E4M3)
    assert np.array_equal(ref, (xi @ wi.T).astype(np.float64))


def test_uniform_block_scales_reduce_to_per_tensor():
    rng = np.random.default_rng(23)
    M, N, K = 8, 256, 384
    xq = _rand_codes(rng, (M, K), E4M3)
    wq = _rand_codes(rng, (N, K), E4M3)
    sx = np.full((M, K // 128), 0.375, np.float32)
    sw = np.full((N // 128, K // 128), 1.25, np.float32)
    a, _ = gemm.gemm_ref(xq, sx, quant.TILE_1x128, E4M3, wq, sw, quant.BLOCK_128x128, E4M3)
    b, _ = gemm.gemm_ref(xq, np.array([0.375], np.float32), quant.TENSOR, E4M3,
                         wq, np.array([1.25], np.float32), quant.TENSOR, E4M3)
    assert np.array_equal(a, b)


def test_mx_unit_exponent_reduces_to_unscaled():
    rng = np.random.default_rng(24)
    M, N, K = 8, 16, 256
    xq = _rand_codes(rng, (M, K), E4M3)
    wq = _rand_codes(rng, (N, K), E5M2)
    ex = np.full((M, K // 32), 127, np.uint8)
    ew = np.full((N, K // 32), 127, np.uint8)
    a, _ = gemm.gemm_ref(xq, ex, quant.MX32, E4M3, wq, ew, quant.MX32, E5M2)
    b = formats.decode(xq, E4M3) @ formats.decode(wq, E5M2).T
    assert np.array_equal(a, b)


def test_blockwise_promotion_identity():
    """sum over 128-K blocks of s_X s_W P_kb equals the GEMM of the dequantized
    operands (the promotion form of the same sum)."""
    rng = np.random.default_rng(25)
    M, N, K = 4, 256, 512
    xq = _rand_codes(rng, (M, K), E4M3)
    wq = _rand_codes(rng, (N, K), E4M3)
    sx = _scales(rng, quant.TILE_1x128, M, K)
    sw = _scales(rng, quant.BLOCK_128x128, N, K)
    ref, absb = gemm.gemm_ref(xq, sx, quant.TILE_1x128, E4M3, wq, sw, quant.BLOCK_128x128, E4M3)
    dx = formats.decode(xq, E4M3)
    dw = formats.decode(wq, E4M3)
    acc = np.zeros((M, N))
    for kb in range(K // 128):
        p = dx[:, kb * 128:(kb + 1) * 128] @ dw[:, kb * 128:(kb + 1) * 128].T
        acc += p * sx[:, kb][:, None] * np.repeat(sw[:, kb], 128)[None, :]
    assert np.all(np.abs(acc - ref) <= 1e-13 * absb)


def test_sampled_pairs_match_full():
    rng = np.random.default_rng(26)
    M, N, K = 32, 256, 256
    xq = _rand_codes(rng, (M, K), E4M3)
    wq = _rand_codes(rng, (N, K), E4M3)
    sx = _scales(rng, quant.TILE_1x128, M, K)
    sw = _scales(rng, quant.BLOCK_128x128, N, K)
    ref, absb = gemm.gemm_ref(xq, sx, quant.TILE_1x128, E4M3, wq, sw, quant.BLOCK_128x128, E4M3)
    mi = rng.integers(0, M, 50)
    ni = rng.integers(0, N, 50)
    xr = gemm.dequant_rows(xq, sx, quant.TILE_1x128, E4M3, np.arange(M))
    wr = gemm.dequant_rows(wq, sw, quant.BLOCK_128x128, E4M3, np.arange(N))
    r, a = gemm.gemm_ref_pairs(xr, wr, mi, ni)
    assert np.allclose(r, ref[mi, ni], rtol=0, atol=1e-12 * absb.max())
    assert np.allclose(a, absb[mi, ni], rtol=1e-14)


def test_tolerance_functions():
    ref = np.array([1.0, -2.0, 0.0, 100.0])
    absb = np.array([10.0, 10.0, 0.0, 200.0])
    ok, _ = gemm.check_f32(np.array([1.0009, -2.001, 0.0, 100.02]), ref, absb)
    assert ok.tolist() == [True, True, True, True]
    ok, _ = gemm.check_f32(np.array([1.0011, -2.0, 1e-30, 100.0201]), ref, absb)
    assert ok.tolist() == [False, True, False, False]
    # bf16 numbers in [64, 128) are spaced 0.5: a reference at the midpoint
    # 100.25 accepts either neighbour (half an ulp), not the one beyond.
    assert gemm.ulp_bf16(np.array([100.0]))[0] == 0.5
    bits = quant.to_bf16_bits(np.array([100.0, 100.5, 101.0], np.float32))
    ok, _ = gemm.check_bf16(bits, np.full(3, 100.25), np.full(3, 1.0))
    assert ok.tolist() == [True, True, False]
    ok, _ = gemm.check_bf16(bits[:1], np.full(1, 100.2600001), np.full(1, 1.0))
    assert ok.tolist() == [False]


def test_worst_case_two_level_bound_fits_tolerance():
    """Two-level accumulation (an exact-enough 128-term block sum, then K/128
    fp32 promotions) is inside 1e-4 * Abs at the largest K of the workloads;
    a single fp32 chain over K terms would not be."""
    K = max(w.K for w in workloads.CONFIGS.values())
    u = 2.0 ** -24
    assert (128 + K / 128 + 3) * u < 1e-4
    assert K * u > 1e-4
