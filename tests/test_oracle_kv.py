"""Pins for the oracle's FP8 KV-cache codec (CPU only): quantize on append,
dequantize on read, scale kinds, slot handling and the cache-size formula."""

import os

import numpy as np
import pytest

from oracle import formats, quant
from oracle.formats import E4M3, E5M2

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _short_scales(rng, n, bits=18):
    """Positive fp32 scales with at most `bits` significant bits, so that any
    FP8 value times the scale is exact in fp32."""
    m = rng.integers(2 ** (bits - 1), 2 ** bits, n).astype(np.float64)
    e = rng.integers(-30, 10, n)
    return np.ldexp(m, e - bits).astype(np.float32)


def _finite_codes(f):
    c = np.arange(256, dtype=np.uint8)
    return c[np.isfinite(formats.decode(c, f))]


def test_cache_size_formula_matches_printed_table():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "kv_cache_memory.txt")) if l.strip() and l[0] != "#"]
    assert len(rows) == 2
    for _, layers, heads, dim, batch, seq, nbytes, gb in rows:
        b = quant.kv_cache_bytes(int(batch), int(seq), int(heads), int(dim), int(nbytes), layers=int(layers))
        assert f"{b / 1e9:.1f}" == gb
    # FP8 halves the bf16 cache exactly
    assert quant.kv_cache_bytes(3, 5, 7, 16, 2) == 2 * quant.kv_cache_bytes(3, 5, 7, 16, 1)


@pytest.mark.parametrize("f", [E4M3, E5M2])
@pytest.mark.parametrize("kind", [quant.KV_SCALE_TENSOR, quant.KV_SCALE_HEAD, quant.KV_SCALE_CHANNEL])
def test_exact_multiples_round_trip(f, kind):
    """x = decode(c) * s is exact in fp32, so x / s = decode(c): append must
    store c itself and the read must give x back bit for bit.  A scale taken
    from the wrong head or channel changes the quotient and the code."""
    rng = np.random.default_rng(7 + kind)
    heads, dim, tokens = 3, 32, 9
    n_sc = {quant.KV_SCALE_TENSOR: 1, quant.KV_SCALE_HEAD: heads, quant.KV_SCALE_CHANNEL: heads * dim}[kind]
    scales = _short_scales(rng, n_sc)
    s = quant.kv_scale_of(kind, scales, heads, dim)
    codes = rng.choice(_finite_codes(f), size=(tokens, heads, dim))
    x = (formats.decode(codes, f) * s.astype(np.float64)).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), formats.decode(codes, f) * s.astype(np.float64))
    slots = rng.permutation(20)[:tokens]
    cache = quant.kv_append(np.zeros((20, heads, dim), np.uint8), x, slots, kind, scales, f)
    assert np.array_equal(cache[slots], codes)
    back = quant.kv_gather(cache, slots, kind, scales, f)
    assert np.array_equal(back.view(np.uint32), x.view(np.uint32))


def test_scale_index_layout():
    """Per head: scale h covers channels [h*D, (h+1)*D); per channel: scale
    h*D + d.  Distinct powers of two per position make every code tell which
    scale it was divided by."""
    heads, dim = 2, 16
    sc = np.ldexp(1.0, np.arange(heads * dim) - 15).astype(np.float32)
    x = np.ones((1, heads, dim), np.float32)
    c = quant.kv_append(np.zeros((1, heads, dim), np.uint8), x, [0], quant.KV_SCALE_CHANNEL, sc, E5M2)
    v = formats.decode(c[0], E5M2)
    assert np.array_equal(v.reshape(-1), 2.0 ** (15 - np.arange(heads * dim)))
    sh = np.array([0.5, 4.0], np.float32)
    c = quant.kv_append(np.zeros((1, heads, dim), np.uint8), x, [0], quant.KV_SCALE_HEAD, sh, E4M3)
    v = formats.decode(c[0], E4M3)
    assert np.all(v[0] == 2.0) and np.all(v[1] == 0.25)


def test_scale_kinds_agree_when_scales_repeat():
    rng = np.random.default_rng(3)
    heads, dim = 4, 16
    x = rng.standard_normal((5, heads, dim)).astype(np.float32) * 3
    base = np.zeros((8, heads, dim), np.uint8)
    slots = [7, 0, 3, 5, 1]
    t = quant.kv_append(base, x, slots, quant.KV_SCALE_TENSOR, [0.013], E4M3)
    h = quant.kv_append(base, x, slots, quant.KV_SCALE_HEAD, np.full(heads, 0.013, np.float32), E4M3)
    assert np.array_equal(t, h)
    sh = np.array([0.01, 0.02, 0.005, 0.3], np.float32)
    h = quant.kv_append(base, x, slots, quant.KV_SCALE_HEAD, sh, E4M3)
    c = quant.kv_append(base, x, slots, quant.KV_SCALE_CHANNEL, np.repeat(sh, dim), E4M3)
    assert np.array_equal(h, c)


def test_power_of_two_scale_is_exact_shift():
    """With s = 2^k, RN32(x / s) = x * 2^-k exactly (normal range), so the code
    is the plain FP8 rounding of x * 2^-k."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((6, 2, 64)) * 40).astype(np.float32)
    for f in (E4M3, E5M2):
        for k in (-3, 0, 5):
            c = quant.kv_append(np.zeros((6, 2, 64), np.uint8), x, np.arange(6), quant.KV_SCALE_TENSOR,
                                [2.0 ** k], f)
            assert np.array_equal(c, formats.encode_nearest(x.astype(np.float64) * 2.0 ** -k, f))


def test_ties_round_to_even():
    """x / s halfway between two E4M3 values goes to the even code: 1.0625
    lies between 1.0 (0x38) and 1.125 (0x39); 1.1875 between 1.125 and 1.25
    (0x3A)."""
    s = np.float32(0.0390625 * 3)           # 3 * 2^-5.xx: few significant bits, products exact
    x = np.array([1.0625, 1.1875, -1.0625], np.float64) * np.float64(s)
    x = x.astype(np.float32).reshape(1, 1, 3)
    x = np.concatenate([x, np.zeros((1, 1, 13), np.float32)], axis=2)
    c = quant.kv_append(np.zeros((1, 1, 16), np.uint8), x, [0], quant.KV_SCALE_TENSOR, [s], E4M3)
    assert list(c[0, 0, :3]) == [0x38, 0x3A, 0xB8]


def test_saturation_even_when_the_quotient_leaves_fp32():
    """clip(round(x / s), -Vmax, Vmax): a quotient beyond Vmax saturates, also
    when it is beyond the fp32 range (E5M2 must not produce its Inf code)."""
    x = np.array([[[1e30, -1e30, 500.0, -500.0] + [0.0] * 12]], np.float32)
    for f, vcode in ((E4M3, 0x7E), (E5M2, 0x7B)):
        c = quant.kv_append(np.zeros((1, 1, 16), np.uint8), x, [0], quant.KV_SCALE_TENSOR, [1e-20], f)
        assert list(c[0, 0, :4]) == [vcode, vcode | 0x80, vcode, vcode | 0x80]
        c = quant.kv_append(np.zeros((1, 1, 16), np.uint8), x, [0], quant.KV_SCALE_TENSOR, [1.0], f)
        v = formats.decode(c[0, 0, 2:4], f)
        assert list(v) == ([448.0, -448.0] if f is E4M3 else [512.0, -512.0])
    # the delayed-scaling quantizer shares the rule
    codes, _, _ = quant.quantize_delayed(np.full((1, 128), 1e30, np.float32), np.array([1e-30], np.float32), 0, 0,
                                         E5M2)
    assert np.all(codes == 0x7B)


def test_slots_outside_the_pool():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 1, 16)).astype(np.float32)
    base = np.full((3, 1, 16), 0x11, np.uint8)
    c = quant.kv_append(base, x, [-1, 3, 1, 1 << 40], quant.KV_SCALE_TENSOR, [0.01], E4M3)
    assert np.array_equal(c[[0, 2]], base[[0, 2]])
    assert np.array_equal(c[1], quant.quantize_with_scale(x[2], np.float32(0.01), E4M3))
    g = quant.kv_gather(c, [-5, 1, 3, 0], quant.KV_SCALE_TENSOR, [0.01], E4M3)
    assert np.all(g[0] == 0) and np.all(g[2] == 0)
    assert np.array_equal(g[3], (formats.decode(base[0], E4M3) * np.float64(np.float32(0.01))).astype(np.float32))
    assert quant.kv_gather(c, np.zeros(0, np.int64), 0, [1.0], E4M3).shape == (0, 1, 16)
