"""FP8 E4M3 / E5M2 decode and the unscaled saturating cast (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Formats, as the pages state them:
  * E4M3: 1 sign, 4 exponent, 3 mantissa bits, bias 7.  Normal values
    (-1)^S * 2^(E-7) * (1 + M/8) for E in 1..15, subnormals (-1)^S * 2^-6 * M/8,
    no infinities, a single NaN magnitude S.1111.111, max 448, min normal 2^-6.
    ("The FP8 Family", section "The two shapes", bit-layout formulas; "FP8
    Mixed-Precision Serving", section "The Mathematics of FP8".)
  * E5M2: 1 sign, 5 exponent, 2 mantissa bits, bias 15, IEEE-like Inf/NaN,
    max 57344, min normal 2^-14 ("The FP8 Family", format table; "FP8
    Mixed-Precision Serving", "Core Architectural Differences").  The pages do
    not write E5M2's subnormal rule; the IEEE rule 2^-14 * M/4 is used, by
    analogy with E4M3's and with the page's remark that E5M2 keeps IEEE
    conventions.
  * Generic value formula x = (-1)^s 2^(e-bias) (1 + sum b_i 2^-i)
    ("FP8 Mixed-Precision Serving", "The Mathematics of FP8").

Cast (fp32 value -> code), "clip(round(x/s), fp8_min, fp8_max)" with s = 1
("The FP8 Family", "Scaling is what makes FP8 usable"; "FP8 Mixed-Precision
Serving", per-tensor scaling formula), rounding to nearest with ties to even
and clamping finite overflow to the format's largest value (the rounding and
saturation modifiers the comments of the qdq listing in "Illustrated GPU
kernels, Part 8" explain):
  * finite |v| > Vmax -> +-Vmax;
  * otherwise the nearest finite code, ties to the even mantissa;
  * the sign is kept, also for zero results (-0 and small negatives -> 0x80);
  * NaN -> 0x7F / 0xFF by sign; +-Inf -> +-Vmax for E4M3 (no Inf code),
    +-Inf (0x7C / 0xFC) for E5M2.
Two encoders compute this independently: a nearest-value search over the
decoded code table, and the "find the binade and round the mantissa to 3 (E4M3)
or 2 (E5M2) bits" method of the page "FP8 Serving" (section "What we can and
cannot measure here").
"""

from __future__ import annotations

import dataclasses
from fractions import Fraction

import numpy as np


@dataclasses.dataclass(frozen=True)
class Fp8Format:
    name: str
    ebits: int
    mbits: int
    bias: int
    has_inf: bool

    @property
    def vmax(self) -> float:
        """Largest finite value, computed from the code table."""
        return float(np.nanmax(np.where(np.isfinite(decode_table(self)), decode_table(self), np.nan)))

    @property
    def emin(self) -> int:
        """Exponent of the smallest normal binade (1 - bias)."""
        return 1 - self.bias


E4M3 = Fp8Format("e4m3", 4, 3, 7, has_inf=False)
E5M2 = Fp8Format("e5m2", 5, 2, 15, has_inf=True)
FORMATS = {0: E4M3, 1: E5M2, "e4m3": E4M3, "e5m2": E5M2}


def fmt_of(f) -> Fp8Format:
    return f if isinstance(f, Fp8Format) else FORMATS[f]


def decode_code(code: int, f) -> float:
    """Value of one code, written out from the bit-layout formulas."""
    f = fmt_of(f)
    s = (code >> 7) & 1
    e = (code >> f.mbits) & ((1 << f.ebits) - 1)
    m = code & ((1 << f.mbits) - 1)
    sign = -1.0 if s else 1.0
    emax_field = (1 << f.ebits) - 1
    if f.has_inf:
        # IEEE-style: the all-ones exponent holds Inf (M = 0) and NaN (M != 0).
        if e == emax_field:
            return sign * float("inf") if m == 0 else float("nan")
    else:
        # E4M3: only S.1111.111 is NaN; the rest of the top binade is normal.
        if e == emax_field and m == (1 << f.mbits) - 1:
            return float("nan")
    if e == 0:
        return sign * 2.0 ** (1 - f.bias) * (m / 2.0 ** f.mbits)
    return sign * 2.0 ** (e - f.bias) * (1.0 + m / 2.0 ** f.mbits)


_TABLE_CACHE: dict = {}


def decode_table(f) -> np.ndarray:
    """fp64 value of every code 0..255."""
    f = fmt_of(f)
    if f.name not in _TABLE_CACHE:
        _TABLE_CACHE[f.name] = np.array([decode_code(c, f) for c in range(256)], dtype=np.float64)
    return _TABLE_CACHE[f.name]


def decode(codes: np.ndarray, f) -> np.ndarray:
    """Decode an array of uint8 codes to fp64 (exact)."""
    return decode_table(f)[np.asarray(codes, dtype=np.uint8)]


def _positive_finite(f):
    """(values, codes) of the non-negative finite codes, ascending."""
    f = fmt_of(f)
    t = decode_table(f)[:128]
    codes = np.array([c for c in range(128) if np.isfinite(t[c])], dtype=np.int64)
    vals = t[codes]
    order = np.argsort(vals, kind="stable")
    return vals[order], codes[order]


def vmax_code(f) -> int:
    vals, codes = _positive_finite(f)
    return int(codes[-1])


def encode_nearest(v, f) -> np.ndarray:
    """Cast fp64-held values (exact fp32 numbers) to codes by nearest-value search."""
    f = fmt_of(f)
    v = np.asarray(v, dtype=np.float64)
    vals, codes = _positive_finite(f)
    a = np.abs(v)
    neg = np.signbit(v)
    finite = np.isfinite(v)
    a_f = np.where(finite, a, 0.0)
    sat = a_f > vals[-1]
    a_c = np.minimum(a_f, vals[-1])
    hi = np.clip(np.searchsorted(vals, a_c, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo = a_c - vals[lo]
    d_hi = vals[hi] - a_c
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi] & 1) == 0) & (hi != lo))
    out = np.where(pick_hi, codes[hi], codes[lo])
    out = np.where(a_c == vals[hi], codes[hi], out)  # exact hits
    out = np.where(sat, codes[-1], out).astype(np.int64)
    # specials
    if f.has_inf:
        inf_code = 0x7C if f.name == "e5m2" else None
        out = np.where(np.isinf(v), inf_code, out)
    else:
        out = np.where(np.isinf(v), codes[-1], out)
    out = np.where(np.isnan(v), 0x7F, out)
    out = out | np.where(neg, 0x80, 0)
    return out.astype(np.uint8)


def round_to_binade(a: np.ndarray, mbits: int, emin: int) -> np.ndarray:
    """Round non-negative finite fp64 values to a floating grid with `mbits`
    fraction bits and smallest normal exponent `emin`, nearest-even, without
    an upper bound: find the binade of each value, then round its mantissa."""
    a = np.asarray(a, dtype=np.float64)
    m, ex = np.frexp(a)            # a = m * 2^ex, m in [0.5, 1)
    e = ex - 1                     # a in [2^e, 2^(e+1))
    e = np.maximum(e, emin)        # below the normal range the quantum is fixed
    quantum = np.ldexp(1.0, e - mbits)
    n = np.rint(a / quantum)       # exact division by a power of two; rint is ties-to-even
    return np.where(a == 0, 0.0, n * quantum)


def encode_binade(v, f) -> np.ndarray:
    """Cast by binade rounding ("FP8 Serving": find the binade, round the
    mantissa to 3 or 2 bits), then saturate and assemble the code bits."""
    f = fmt_of(f)
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    finite = np.isfinite(v)
    a = np.where(finite, np.abs(v), 0.0)
    # the largest finite value from the bit layout (not from the code table)
    top_e = (1 << f.ebits) - 1 - f.bias if not f.has_inf else (1 << f.ebits) - 2 - f.bias
    top_m = (1 << f.mbits) - 2 if not f.has_inf else (1 << f.mbits) - 1
    vmax = 2.0 ** top_e * (1 + top_m / 2.0 ** f.mbits)
    r = round_to_binade(a, f.mbits, f.emin)
    r = np.minimum(r, vmax)
    mant, ex = np.frexp(r)
    e = ex - 1
    sub = (r < 2.0 ** f.emin)
    e_field = np.where(sub, 0, e + f.bias)
    m_field = np.where(sub,
                       np.rint(r / 2.0 ** (f.emin - f.mbits)),
                       np.rint((r / np.ldexp(1.0, e) - 1.0) * 2 ** f.mbits))
    code = (e_field.astype(np.int64) << f.mbits) | m_field.astype(np.int64)
    code = np.where(r == 0, 0, code)
    if f.has_inf:
        code = np.where(np.isinf(v), ((1 << f.ebits) - 1) << f.mbits, code)
    else:
        code = np.where(np.isinf(v), (top_e + f.bias) << f.mbits | top_m, code)
    code = np.where(np.isnan(v), 0x7F, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


# The oracle's cast: the nearest-value encoder (the binade encoder is its pin).
encode = encode_nearest


def round_exact_fraction(x: Fraction, f) -> int:
    """Encode one exact rational by brute force over all non-negative codes
    (nearest to |x|, ties to the even mantissa, then saturating by
    construction since Vmax is the nearest code above it); tiny-case pin."""
    f = fmt_of(f)
    t = decode_table(f)
    ax = abs(x)
    best = None
    for c in range(128):
        val = t[c]
        if not np.isfinite(val):
            continue
        key = (abs(Fraction(val) - ax), c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    c = best[1]
    return c | 0x80 if x < 0 else c
