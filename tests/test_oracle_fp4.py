"""Pins for the oracle's FP4 (E2M1) microscaling: the element grid, the cast,
MXFP4 and NVFP4 scales, quantize/dequantize and the GEMM reference (CPU only)."""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats, fp4
from oracle.formats import E4M3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rn32_exact(q: Fraction) -> np.float32:
    """An exact rational rounded to fp32 (nearest, ties to even) by comparing
    exact distances to the neighbouring fp32 numbers."""
    f = np.float32(float(q))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        if not np.isfinite(c):
            continue
        key = (abs(Fraction(float(c)) - q), int(np.array(c).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_e2m1_grid_is_the_two_bit_part_of_e4m3():
    """E2M1 magnitudes are exactly the E4M3 values up to 6 that sit on a grid
    with one mantissa bit and smallest normal binade [1, 2): a multiple of 0.5
    below 1, of half the binade's power of two above (E4M3's table is pinned
    on its own)."""
    e4 = formats.decode(np.arange(128, dtype=np.uint8), E4M3)
    e4 = e4[np.isfinite(e4)]

    def on_grid(v):
        if v == 0:
            return True
        quantum = 0.5 if v < 1 else 2.0 ** np.floor(np.log2(v)) / 2
        return v <= 6 and v % quantum == 0

    assert sorted(set(v for v in e4 if on_grid(v))) == list(fp4.E2M1_TABLE[:8])
    assert np.array_equal(fp4.E2M1_TABLE[8:], -fp4.E2M1_TABLE[:8])
    assert np.signbit(fp4.E2M1_TABLE[8])


def test_cast_ties_and_saturation():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_ties.txt")) if l.strip() and l[0] != "#"]
    v = np.array([float(a) for a, _ in rows])
    want = np.array([int(b) for _, b in rows], np.uint8)
    assert np.array_equal(fp4.e2m1_encode_nearest(v), want)
    assert np.array_equal(fp4.e2m1_encode_binade(v), want)


def test_two_encoders_agree_densely():
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.uniform(-8, 8, 200000), rng.standard_normal(50000) * 1e-3,
                        np.arange(-7, 7.01, 0.125), fp4.E2M1_TABLE])
    assert np.array_equal(fp4.e2m1_encode_nearest(v), fp4.e2m1_encode_binade(v))
    # every code casts back to itself
    assert np.array_equal(fp4.e2m1_encode_nearest(fp4.E2M1_TABLE), np.arange(16, dtype=np.uint8))


def test_pack_nibble_order():
    c = np.array([[1, 2, 0xF, 0x8]], np.uint8)
    p = fp4.pack(c)
    assert list(p[0]) == [0x21, 0x8F]
    assert np.array_equal(fp4.unpack(p), c)


def test_mx_exponent_exact():
    rng = np.random.default_rng(8)
    m = rng.integers(2 ** 23, 2 ** 24, 3000)
    ex = rng.integers(-140, 120, 3000)
    amax = np.ldexp(m.astype(np.float64), ex - 23).astype(np.float32)
    amax = np.concatenate([amax, np.float32([6, 12, 3, 6 * 2.0 ** -127, 6 * 2.0 ** -128, 0])])
    got = fp4.mx_exponent(amax.astype(np.float64))
    for a, e in zip(amax, got):
        a = Fraction(float(a))
        if a == 0:
            assert e == -127
            continue
        want = -127
        while want < 127 and a > 6 * Fraction(2) ** want:
            want += 1
        if want == -127 and a <= 6 * Fraction(2) ** -127:
            want = -127
        assert e == want, (a, e, want)


def test_mx_quantize_invariants_and_exact_round_trip():
    rng = np.random.default_rng(9)
    # blocks of exact multiples: codes with one +-6 per block and a power-of-two scale
    rows, K = 5, 128
    e = rng.integers(-20, 20, (rows, K // 32))
    codes = rng.integers(0, 16, (rows, K)).astype(np.uint8)
    codes[:, ::32] = np.where(rng.integers(0, 2, (rows, K // 32)) == 1, 7, 15)
    x = (fp4.e2m1_decode(codes).reshape(rows, K // 32, 32) * np.ldexp(1.0, e)[..., None]).reshape(rows, K)
    q, s = fp4.quantize_mx(x.astype(np.float32))
    assert np.array_equal(s.astype(np.int64) - 127, e)
    assert np.array_equal(fp4.unpack(q), codes)
    assert np.array_equal(fp4.dequantize_mx(q, s), x.astype(np.float32))
    # random data: no element saturates and every block's largest lands in the top binade
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-6, 6, (64, 1)))).astype(np.float32)
    q, s = fp4.quantize_mx(x)
    ee = s.astype(np.int64) - 127
    scaled = np.abs(x.reshape(64, 8, 32)) * np.ldexp(1.0, -ee)[..., None]
    assert scaled.max() <= 6
    assert np.all(scaled.max(axis=2) > 3)


def test_nv_scales_step_by_step():
    """Each NVFP4 rounding against exact rationals, and the tensor's largest
    block landing on 448, the top of E4M3."""
    rng = np.random.default_rng(10)
    x = (rng.standard_normal((32, 128)) * np.exp(rng.uniform(-3, 3, (32, 8))).repeat(16, axis=1)).astype(np.float32)
    q, m, s_t = fp4.quantize_nv(x)
    amax_t = Fraction(float(np.abs(x).max()))
    assert s_t == rn32_exact(amax_t / 2688)
    t = rn32_exact(Fraction(float(s_t)) * 6)
    amax_b = np.abs(x.reshape(32, 8, 16)).max(axis=2)
    for r in range(32):
        for b in range(8):
            u = rn32_exact(Fraction(float(amax_b[r, b])) / Fraction(float(t)))
            assert m[r, b] == formats.encode(np.float64(u), E4M3)
    top = np.unravel_index(np.argmax(amax_b), amax_b.shape)
    assert m[top] == 0x7E and formats.decode(m, E4M3).max() == 448
    # the effective scale and the codes of a few blocks, from Fractions
    S = fp4.nv_effective_scales(m, s_t)
    codes = fp4.unpack(q)
    for r, b in [(0, 0), (5, 3), (31, 7)]:
        assert S[r, b] == rn32_exact(Fraction(float(formats.decode_code(int(m[r, b]), E4M3))) * Fraction(float(s_t)))
        for k in range(16):
            qv = rn32_exact(Fraction(float(x[r, 16 * b + k])) / Fraction(float(S[r, b])))
            assert codes[r, 16 * b + k] == fp4.e2m1_encode_nearest(np.float64(qv))


def test_nv_tiny_block_and_zero_tensor():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1000.0
    x[0, 16:] = [1e-9, -1e-9] * 8           # microscale rounds to 0: codes are signed zeros
    q, m, s_t = fp4.quantize_nv(x)
    c = fp4.unpack(q)[0]
    assert m[0, 1] == 0 and list(c[16:18]) == [0, 8]
    q, m, s_t = fp4.quantize_nv(np.zeros((2, 16), np.float32))
    assert s_t == 1.0 and not fp4.unpack(q).any() and not m.any()


def _e2m1_bits_value(code: int) -> Fraction:
    """E2M1 nibble -> exact value from its bit fields (bias 1, subnormal 0.5)."""
    e, m = (code >> 1) & 3, code & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return -mag if code & 8 else mag


def _e4m3_bits_value(code: int):
    """E4M3 byte -> exact value from its bit fields, or None for NaN (S.1111.111)."""
    e, m = (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return None
    mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else Fraction(2) ** (e - 7) * (1 + Fraction(m, 8))
    return -mag if code & 0x80 else mag


def test_dequantize_nv_against_fractions():
    """dequantize_nv element by element against an independent decode: every
    E2M1 code under every E4M3 microscale code (NaN, +-0 and subnormal
    microscales included) and four tensor scales, with S = RN32(m * s_t) and
    y = RN32(q * S) rounded from exact rationals; NaN where the microscale is
    NaN, and the sign of a zero result is the sign of q * S."""
    codes = np.arange(16, dtype=np.uint8)
    for s_t in (np.float32(1.0), np.float32(3.0517578e-05), np.float32(0.0123456789), np.float32(7.25e+30)):
        micro = np.arange(256, dtype=np.uint8).reshape(16, 16)          # 16 rows x 16 blocks: every code
        rows, nblk = micro.shape
        q = np.tile(codes, (rows, nblk))                                # each block holds the 16 codes
        y = fp4.dequantize_nv(fp4.pack(q), micro, s_t)
        assert y.dtype == np.float32 and y.shape == (rows, 16 * nblk)
        for r in range(rows):
            for b in range(nblk):
                mv = _e4m3_bits_value(int(micro[r, b]))
                for k in range(16):
                    got = y[r, 16 * b + k]
                    if mv is None:
                        assert np.isnan(got)
                        continue
                    S = rn32_exact(mv * Fraction(float(s_t)))
                    qv = _e2m1_bits_value(int(q[r, 16 * b + k]))
                    want = rn32_exact(qv * Fraction(float(S)))
                    if want == 0:
                        # zero microscale codes carry their sign into S (s_t > 0 here)
                        s_neg = bool(micro[r, b] & 0x80) if mv == 0 else bool(S < 0)
                        neg = (int(q[r, 16 * b + k]) >= 8) != s_neg
                        assert got == 0 and bool(np.signbit(got)) == neg, (r, b, k)
                    else:
                        assert got.view(np.uint32) == want.view(np.uint32), (r, b, k, got, want)


def test_nv_exact_multiples_round_trip():
    """x built as exact multiples q * m * s_t (s_t a power of two, every block
    holding a +-6 code, the largest microscale 448) quantizes back to the same
    codes, microscales and tensor scale, and dequantizes to x bit for bit."""
    rng = np.random.default_rng(11)
    rows, nblk = 8, 12
    s_t = np.float32(2.0 ** -9)
    mags = [0.5, 1, 1.5, 2, 3, 4, 6]
    micro_vals = [Fraction(v) for v in (448, 0.25, 1.125, 3.5, 40, 96, 240, 0.015625)]
    x = np.zeros((rows, 16 * nblk), np.float32)
    want_m = np.zeros((rows, nblk), np.uint8)
    for r in range(rows):
        for b in range(nblk):
            mv = micro_vals[(r * nblk + b) % len(micro_vals)] if (r, b) != (0, 0) else Fraction(448)
            want_m[r, b] = formats.encode(np.float64(float(mv)), E4M3)
            q = rng.choice(mags, 16) * rng.choice([-1.0, 1.0], 16)
            q[rng.integers(16)] = 6.0 * rng.choice([-1.0, 1.0])
            for k in range(16):
                x[r, 16 * b + k] = np.float32(float(Fraction(q[k]) * mv * Fraction(float(s_t))))
    packed, m, st = fp4.quantize_nv(x)
    assert st == s_t and np.array_equal(m, want_m)
    y = fp4.dequantize_nv(packed, m, st)
    assert np.array_equal(y.view(np.uint32), x.view(np.uint32))


@pytest.mark.parametrize("kind", [fp4.MX, fp4.NV])
def test_gemm_ref_matches_fractions(kind):
    rng = np.random.default_rng(11 + kind)
    M, N, K = 3, 4, 64
    x = (rng.standard_normal((M, K)) * np.exp(rng.uniform(-4, 4, (M, K)))).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    if kind == fp4.MX:
        a, sa = fp4.quantize_mx(x)
        b, sb = fp4.quantize_mx(w)
        ta = tb = None
    else:
        a, sa, ta = fp4.quantize_nv(x)
        b, sb, tb = fp4.quantize_nv(w)
    ref, absb = fp4.gemm_ref(kind, a, sa, b, sb, ta, tb)
    exact = fp4.gemm_exact_fraction(kind, a, sa, b, sb, ta, tb)
    for i in range(M):
        for j in range(N):
            assert abs(Fraction(float(ref[i, j])) - exact[i][j]) <= Fraction(1, 10 ** 12) * Fraction(float(absb[i, j])) + Fraction(1, 10 ** 300)


def test_gemm_special_cases():
    """MX with every scale 2^0 is the plain E2M1 matmul; NV with unit
    microscales and tensor scales likewise."""
    rng = np.random.default_rng(12)
    qa = rng.integers(0, 16, (4, 64)).astype(np.uint8)
    qb = rng.integers(0, 16, (5, 64)).astype(np.uint8)
    plain = fp4.e2m1_decode(qa) @ fp4.e2m1_decode(qb).T
    ref, _ = fp4.gemm_ref(fp4.MX, fp4.pack(qa), np.full((4, 2), 127, np.uint8), fp4.pack(qb),
                          np.full((5, 2), 127, np.uint8))
    assert np.array_equal(ref, plain)
    one = formats.encode(np.float64(1.0), E4M3)
    ref, _ = fp4.gemm_ref(fp4.NV, fp4.pack(qa), np.full((4, 4), one, np.uint8), fp4.pack(qb),
                          np.full((5, 4), one, np.uint8), np.float32(1), np.float32(1))
    assert np.array_equal(ref, plain)
