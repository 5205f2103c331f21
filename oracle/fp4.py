"""FP4 (E2M1) with two-level microscaling: MXFP4 and NVFP4 (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is computed, with where the pages say it:
  * "Illustrated GPU kernels, Part 8" (section "Low precision: FP8, FP4, and
    microscaling"): FP4 halves the bytes of FP8 again; the OCP Microscaling
    (MX) format is 32 consecutive elements sharing one UE8M0 scale (a pure
    power of two); NVFP4 uses blocks of 16 with a two-level scale: an E4M3
    microscale per block plus one FP32 scale per tensor "that keeps those
    microscales inside E4M3's own range".
  * The element format is E2M1, the FP4 of the OCP MX specification the page
    cites (the pages do not write its bits out; reading F1): 1 sign, 2
    exponent, 1 mantissa bit, bias 1, from the generic value formula
    x = (-1)^s 2^(e-bias) (1 + m/2) ("FP8 Mixed-Precision Serving", "The
    Mathematics of FP8") with IEEE-style subnormals 2^0 * m/2 for e = 0 and no
    Inf or NaN codes: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
  * The cast is the FP8 one: round to nearest even, finite overflow saturates
    to +-6, the sign of zero results is kept ("Part 8", qdq listing comments).
  * Packing (reading F2): two codes per byte, element 2i in the low nibble,
    element 2i+1 in the high nibble; a row of K elements is K/2 bytes.
  * MXFP4 (reading F3): per 32 elements, e = the smallest integer with
    amax <= 6 * 2^e, clamped to [-127, 127] (-127 for an all-zero block) --
    the same rule as the FP8 MX32 scale, with 6 as the element maximum; the
    scale byte is e + 127; codes = cast(x * 2^-e).
  * NVFP4 (reading F4), every rounding explicit:
      s_t = RN32(amax_tensor / 2688)  (2688 = 6 * 448), 1 when that is 0
      per 16 elements:  t = RN32(6 * s_t);  u = RN32(amax_block / t)
                        m = E4M3 code of u (round to nearest even, saturating)
                        S = RN32(decode(m) * s_t)       the block's fp32 scale
      codes = cast(RN32(x / S)); all +-0 (sign of x) when S == 0.
    The largest block's microscale is then 448, the top of E4M3.
  * Dequantize: MX  decode(q) * 2^e;  NV  RN32(decode(q) * S).
  * GEMM: Out[m, n] = sum_k deq(a[m, k]) deq(b[n, k]) with the two-level scale
    applied as the product it is: MX sum_k qa 2^ea qb 2^eb; NV
    s_ta s_tb sum_k (qa ma)(qb mb) (ma, mb the E4M3 microscale values).
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

from . import formats

MX, NV = 0, 1
MX_BLOCK, NV_BLOCK = 32, 16
VMAX = 6.0
NV_TENSOR_DIVISOR = 6.0 * 448.0      # 2688: E2M1 max times E4M3 max


# ---- E2M1 ----------------------------------------------------------------------

def e2m1_value(code: int) -> float:
    """Value of a 4-bit code, from the bit layout."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    sign = -1.0 if s else 1.0
    if e == 0:
        return sign * (m / 2.0)
    return sign * 2.0 ** (e - 1) * (1.0 + m / 2.0)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e2m1_decode(codes) -> np.ndarray:
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def e2m1_encode_nearest(v) -> np.ndarray:
    """Cast fp64-held values to 4-bit codes: nearest magnitude, ties to the
    even code, saturating at 6, sign kept."""
    v = np.asarray(v, dtype=np.float64)
    mags = E2M1_TABLE[:8]                       # 0, .5, 1, 1.5, 2, 3, 4, 6 (codes 0..7)
    a = np.minimum(np.abs(v), VMAX)
    d = np.abs(a[..., None] - mags)             # distance to every magnitude
    best = np.argmin(d, axis=-1)
    # ties: argmin returns the lower code; take the even one of the pair
    dmin = np.take_along_axis(d, best[..., None], -1)[..., 0]
    nxt = np.minimum(best + 1, 7)
    tie = (np.take_along_axis(d, nxt[..., None], -1)[..., 0] == dmin) & (nxt != best)
    code = np.where(tie & (best % 2 == 1), nxt, best)
    return (code | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def e2m1_encode_binade(v) -> np.ndarray:
    """The same cast by binade rounding: round the mantissa to 1 bit in the
    value's binade (fixed quantum 0.5 below 1), clamp at 6, assemble bits."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    r = np.minimum(formats.round_to_binade(a, 1, 0), VMAX)
    mant, ex = np.frexp(r)                      # r = mant * 2^ex, mant in [0.5, 1)
    e = ex - 1
    sub = r < 1.0
    e_field = np.where(sub, 0, e + 1)
    m_field = np.where(sub, np.rint(r / 0.5), np.rint((r / np.ldexp(1.0, e) - 1.0) * 2))
    code = (e_field.astype(np.int64) << 1) | m_field.astype(np.int64)
    code = np.where(r == 0, 0, code)
    return (code | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def pack(codes: np.ndarray) -> np.ndarray:
    """[rows, K] 4-bit codes -> [rows, K/2] bytes (element 2i low nibble)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ---- MXFP4 -----------------------------------------------------------------------

def mx_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest e with amax <= 6 * 2^e, clamped to [-127, 127]; -127 for 0."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    # 6 * 2^e >= amax  <=>  e >= log2(amax / 6); found exactly with frexp
    m, ex = np.frexp(np.where(nz, amax, 1.0) / VMAX)   # amax/6 = m 2^ex, m in [0.5, 1)
    e = np.where(m == 0.5, ex - 1, ex)                 # exact powers of two need no extra binade
    out = np.where(nz, np.clip(e, -127, 127), out)
    return out


def quantize_mx(x: np.ndarray):
    """x [rows, K] (K % 32 == 0) -> (packed codes [rows, K/2], scale bytes [rows, K/32])."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    rows, K = x64.shape
    blocks = x64.reshape(rows, K // MX_BLOCK, MX_BLOCK)
    e = mx_exponent(np.abs(blocks).max(axis=2))
    q = e2m1_encode_nearest(blocks * np.ldexp(1.0, -e)[..., None]).reshape(rows, K)
    return pack(q), (e + 127).astype(np.uint8)


def dequantize_mx(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """decode(q) * 2^e; a scale byte of 255 (never written) reads as NaN, as for
    the FP8 MX32 scale."""
    q = unpack(packed)
    rows, K = q.shape
    b = np.asarray(scales, dtype=np.int64)
    e = np.minimum(b, 254) - 127
    v = e2m1_decode(q).reshape(rows, K // MX_BLOCK, MX_BLOCK) * np.ldexp(1.0, e)[..., None]
    v = np.where((b == 255)[..., None], np.nan, v)
    with np.errstate(over="ignore"):
        return v.reshape(rows, K).astype(np.float32)


# ---- NVFP4 -----------------------------------------------------------------------

def _rn32(v) -> np.ndarray:
    """Round fp64 values holding an exact product or quotient of fp32 numbers to
    fp32 (the fp64 rounding of such a quotient cannot change the fp32 one: 53 >=
    2 * 24 + 2)."""
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float32)


def nv_tensor_scale(amax: float) -> np.float32:
    s = _rn32(np.float64(np.float32(amax)) / NV_TENSOR_DIVISOR)
    return np.float32(1.0) if s == 0 else np.float32(s)


def nv_block_scales(amax_blocks: np.ndarray, s_t):
    """(microscale E4M3 codes, effective fp32 block scales S) for block amaxes."""
    s_t = np.float32(s_t)
    t = _rn32(np.float64(s_t) * 6.0)
    u = _rn32(np.asarray(amax_blocks, np.float32).astype(np.float64) / np.float64(t))
    m = formats.encode(u.astype(np.float64), formats.E4M3)
    S = _rn32(formats.decode(m, formats.E4M3) * np.float64(s_t))
    return m, S


def quantize_nv(x: np.ndarray):
    """x [rows, K] (K % 16 == 0) -> (packed codes [rows, K/2], microscale codes
    [rows, K/16], tensor scale fp32)."""
    x32 = np.asarray(x, dtype=np.float32)
    rows, K = x32.shape
    s_t = nv_tensor_scale(np.abs(x32).max() if x32.size else 0.0)
    blocks = x32.reshape(rows, K // NV_BLOCK, NV_BLOCK).astype(np.float64)
    m, S = nv_block_scales(np.abs(blocks).max(axis=2).astype(np.float32), s_t)
    S64 = S.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q32 = (blocks / np.where(S64 == 0, 1.0, S64)).astype(np.float32)
    big = np.float32(np.finfo(np.float32).max)     # an fp32-overflowing quotient saturates (reading G21)
    q32 = np.where(np.isinf(q32), np.where(q32 < 0, -big, big), q32)
    codes = e2m1_encode_nearest(q32.astype(np.float64))
    zero = np.where(np.signbit(blocks), 8, 0).astype(np.uint8)
    codes = np.where(S64 == 0, zero, codes).reshape(rows, K)
    return pack(codes), m.astype(np.uint8), np.float32(s_t)


def nv_effective_scales(micro: np.ndarray, s_t) -> np.ndarray:
    return _rn32(formats.decode(micro, formats.E4M3) * np.float64(np.float32(s_t)))


def dequantize_nv(packed: np.ndarray, micro: np.ndarray, s_t) -> np.ndarray:
    q = unpack(packed)
    rows, K = q.shape
    S = nv_effective_scales(micro, s_t).astype(np.float64)
    v = e2m1_decode(q).reshape(rows, K // NV_BLOCK, NV_BLOCK) * S[..., None]
    return _rn32(v.reshape(rows, K))


# ---- GEMM reference ------------------------------------------------------------

def dequant_exact(kind: int, packed, scales, s_t=None) -> np.ndarray:
    """fp64 values whose products are the GEMM's terms: MX q * 2^e (exact);
    NV q * m, the microscale value (the tensor scale applied outside)."""
    q = e2m1_decode(unpack(packed))
    rows, K = q.shape
    if kind == MX:
        e = np.asarray(scales, dtype=np.int64) - 127
        return (q.reshape(rows, K // MX_BLOCK, MX_BLOCK) * np.ldexp(1.0, e)[..., None]).reshape(rows, K)
    m = formats.decode(scales, formats.E4M3)
    return (q.reshape(rows, K // NV_BLOCK, NV_BLOCK) * m[..., None]).reshape(rows, K)


def _scalar32(v) -> np.float32:
    return np.float32(np.asarray(v, dtype=np.float32).reshape(-1)[0])


def gemm_ref(kind: int, a, sa, b, sb, ta=None, tb=None):
    """(Ref, Abs) in fp64: Ref = sum_k deq(a) deq(b) (NV: times s_ta s_tb),
    Abs = the same sum of absolute values (the tolerance's scale)."""
    xa = dequant_exact(kind, a, sa)
    xb = dequant_exact(kind, b, sb)
    ref = xa @ xb.T
    absb = np.abs(xa) @ np.abs(xb).T
    if kind == NV:
        t = float(_scalar32(ta)) * float(_scalar32(tb))
        ref, absb = ref * t, absb * t
    return ref, absb


def gemm_exact_fraction(kind: int, a, sa, b, sb, ta=None, tb=None):
    """Brute-force rational GEMM for tiny shapes (pins gemm_ref)."""
    qa, qb = unpack(a), unpack(b)
    M, K = qa.shape
    N = qb.shape[0]
    blk = MX_BLOCK if kind == MX else NV_BLOCK

    def val(q, s, r, k):
        v = Fraction(e2m1_value(int(q[r, k])))
        if kind == MX:
            return v * Fraction(2) ** (int(s[r, k // blk]) - 127)
        return v * Fraction(float(formats.decode_code(int(s[r, k // blk]), formats.E4M3)))

    out = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += val(qa, sa, i, k) * val(qb, sb, j, k)
            if kind == NV:
                acc *= Fraction(float(_scalar32(ta))) * Fraction(float(_scalar32(tb)))
            out[i][j] = acc
    return out
