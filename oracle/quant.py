"""Scale granularities, amax, scale rules, quantize and dequantize (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is computed, with where the pages say it:
  * quantize  x_fp8 = clip(round(x / s), -Vmax, Vmax); dequantize x_hat = x_fp8 * s
    ("The FP8 Family", section "Scaling is what makes FP8 usable", first two
    formulas; "FP8 Mixed-Precision Serving", per-tensor static scaling formula
    and the block-wise formula in "Block-Wise and Tile Scaling").
  * the scale comes from the group's amax: s = max|x| / Vmax, Vmax = 448 for
    E4M3 ("FP8 Mixed-Precision Serving", the s formula and the block formula;
    "Illustrated GPU kernels, Part 8", qdq listing comment "s = amax / 448").
    It is the current-scaling rule: amax of this tensor, this pass ("FP8
    Mixed-Precision Serving", "Just-in-Time Current Scaling"; "Part 8",
    the NVIDIA taxonomy list).
  * groups ("The FP8 Family", scaling granularity table and the DeepSeek-V3
    callout; "Part 8" taxonomy list and the OCP MX paragraph):
      TENSOR         one fp32 scale for the whole tensor
      ROW            one fp32 per row of a [rows, K] operand (per-token for X,
                     per-output-channel for W stored [N, K])
      TILE_1x128     one fp32 per row x 128 consecutive columns; [rows, K/128]
      BLOCK_128x128  one fp32 per 128 x 128 block; [rows/128, K/128]
      MX32           one UE8M0 byte per row x 32 consecutive columns; [rows, K/32]
  * UE8M0 scale: eight exponent bits, no mantissa, a pure power of two ("Part 8",
    OCP MX paragraph).  The pages give no rule for choosing the exponent.  The
    reading taken: the smallest power of two 2^e with amax <= Vmax * 2^e, so the
    block's largest element falls in the format's top binade, as the pages ask
    of a well-chosen scale ("Part 8", the paragraph before the qdq listing), and
    no element saturates.  The byte is
    e + 127 with e clamped to [-127, 127]; byte 255 is never produced and
    decodes to NaN.
  * amax = 0 (or amax / Vmax rounding to 0 in fp32): s = 1.0, MX e = -127; all
    codes are then +-0.  (The pages do not say; plainest reading.)
  * the division x / s is the correctly rounded fp32 quotient (the formulas
    divide; the listing's multiply by 1/s is a different rounding and is not
    the definition used here).
  * rows, K must be positive multiples as the layouts need: K % 128 == 0 in all
    modes, rows % 128 == 0 for BLOCK_128x128 (partial groups are rejected).
  * with a given scale (delayed scaling, the KV cache) the quotient x / s can
    exceed the fp32 range; clip(round(x / s)) then still saturates to +-Vmax.
"""

from __future__ import annotations

import numpy as np

from . import formats

TENSOR, ROW, TILE_1x128, BLOCK_128x128, MX32 = 0, 1, 2, 3, 4
GRAN_NAMES = {TENSOR: "tensor", ROW: "row", TILE_1x128: "tile_1x128",
              BLOCK_128x128: "block_128x128", MX32: "mx32"}


def scale_shape(gran: int, rows: int, cols: int):
    if gran == TENSOR:
        return (1,)
    if gran == ROW:
        return (rows,)
    if gran == TILE_1x128:
        return (rows, cols // 128)
    if gran == BLOCK_128x128:
        return (rows // 128, cols // 128)
    if gran == MX32:
        return (rows, cols // 32)
    raise ValueError(gran)


def check_shape(gran: int, rows: int, cols: int):
    if cols % 128:
        raise ValueError("K must be a multiple of 128")
    if gran == BLOCK_128x128 and rows % 128:
        raise ValueError("rows must be a multiple of 128 for 128x128 blocks")


def group_amax(x: np.ndarray, gran: int) -> np.ndarray:
    """max |x| over each group, shaped like the scale array (fp64, exact)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    rows, cols = a.shape
    if gran == TENSOR:
        return np.array([a.max() if a.size else 0.0])
    if gran == ROW:
        return a.max(axis=1) if cols else np.zeros(rows)
    if gran == TILE_1x128:
        return a.reshape(rows, cols // 128, 128).max(axis=2)
    if gran == BLOCK_128x128:
        return a.reshape(rows // 128, 128, cols // 128, 128).max(axis=(1, 3))
    if gran == MX32:
        return a.reshape(rows, cols // 32, 32).max(axis=2)
    raise ValueError(gran)


def fp32_scale(amax: np.ndarray, fmt) -> np.ndarray:
    """s = RN32(amax / Vmax); s = 1 where that is 0."""
    f = formats.fmt_of(fmt)
    s = (np.asarray(amax, dtype=np.float64) / f.vmax).astype(np.float32)
    return np.where(s == 0, np.float32(1.0), s).astype(np.float32)


def mx_exponent(amax: np.ndarray, fmt) -> np.ndarray:
    """Smallest integer e with amax <= Vmax * 2^e, from the bits of amax.

    amax = 1.f * 2^E; Vmax = mv * 2^emax with mv in [1, 2).  Then
    e = E - emax when 1.f <= mv, else E - emax + 1; clamped to [-127, 127];
    amax = 0 gives -127."""
    f = formats.fmt_of(fmt)
    amax = np.asarray(amax, dtype=np.float64)
    mv2, emax1 = np.frexp(f.vmax)      # vmax = mv2 * 2^emax1, mv2 in [0.5, 1)
    m2, e1 = np.frexp(amax)            # amax = m2 * 2^e1
    e = np.where(m2 <= mv2, e1 - emax1, e1 - emax1 + 1)
    e = np.where(amax == 0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def broadcast_scale(scales: np.ndarray, gran: int, rows: int, cols: int) -> np.ndarray:
    """Per-element fp64 scale (fp32 scales) or 2^e (MX bytes) for a [rows, cols] operand."""
    if gran == MX32:
        b = np.asarray(scales, dtype=np.int64).reshape(rows, cols // 32)
        val = np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))
        return np.repeat(val, 32, axis=1)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    if gran == TENSOR:
        return np.full((rows, cols), s.reshape(-1)[0])
    if gran == ROW:
        return np.repeat(s.reshape(rows, 1), cols, axis=1)
    if gran == TILE_1x128:
        return np.repeat(s.reshape(rows, cols // 128), 128, axis=1)
    if gran == BLOCK_128x128:
        s2 = s.reshape(rows // 128, cols // 128)
        return np.repeat(np.repeat(s2, 128, axis=0), 128, axis=1)
    raise ValueError(gran)


def quantize(x: np.ndarray, gran: int, fmt):
    """Quantize a [rows, cols] operand given as exact fp32 values.

    Returns (codes uint8 [rows, cols], scales): float32 scales shaped
    scale_shape(...), or uint8 UE8M0 bytes for MX32."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    check_shape(gran, rows, cols)
    amax = group_amax(x, gran)
    x64 = x.astype(np.float64)
    if gran == MX32:
        e = mx_exponent(amax, fmt)
        scaled = x64 * np.repeat(np.ldexp(1.0, -e), 32, axis=1)   # exact power-of-two scaling
        codes = formats.encode(scaled, fmt)
        return codes, (e + 127).astype(np.uint8)
    s = fp32_scale(amax, fmt)
    sb = broadcast_scale(s, gran, rows, cols)
    q32 = (x64 / sb).astype(np.float32)           # correctly rounded fp32 x / s
    codes = formats.encode(q32.astype(np.float64), fmt)
    return codes, s.reshape(scale_shape(gran, rows, cols))


def dequantize(codes: np.ndarray, scales: np.ndarray, gran: int, fmt) -> np.ndarray:
    """y = RN32(decode(q) * s) (MX: decode(q) * 2^e), as float32."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, cols = codes.shape
    v = formats.decode(codes, fmt) * broadcast_scale(scales, gran, rows, cols)
    with np.errstate(over="ignore", invalid="ignore"):
        return v.astype(np.float32)


def to_bf16_bits(y: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even; overflow to Inf) by
    binade rounding with 7 fraction bits; returns uint16 bit patterns."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    fin = np.isfinite(a)
    r = formats.round_to_binade(np.where(fin, a, 0.0), 7, -126)
    r = np.where(fin, r, a)
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)            # exact: r has <= 8 significant bits
    r32 = np.where(r >= 2.0 ** 128, np.float32(np.inf), r32)
    bits = (r32.view(np.uint32) >> 16).astype(np.uint16)
    bits = bits | np.where(np.signbit(y), 0x8000, 0).astype(np.uint16)
    return np.where(np.isnan(y), np.uint16(0x7FC0), bits).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---- delayed scaling --------------------------------------------------------
# "FP8 Mixed-Precision Serving", section "Quantization Granularity and Scaling
# Topologies", delayed scaling: the scale of a per-tensor quantization comes
# from a rolling history H of the amax of earlier iterations (length l, e.g.
# 1024), rho = FP8max / (2^m max(H)) with a safety margin m, instead of from the
# current tensor; the current tensor's amax then enters the history.  Stored
# as the dequant multiplier s = 1 / rho = 2^m max(H) / Vmax (reading G2).


def delayed_scale(history: np.ndarray, margin: int, fmt) -> np.float32:
    """s = RN32(2^m * max(H) / Vmax), 1 when that is 0; NaN entries are ignored."""
    h = np.asarray(history, dtype=np.float32).astype(np.float64).reshape(-1)
    h = h[~np.isnan(h)]
    amax = float(h.max()) if h.size else 0.0
    f = formats.fmt_of(fmt)
    with np.errstate(over="ignore"):
        s = np.float32(np.ldexp(amax, margin) / f.vmax)
    return np.float32(1.0) if s == 0 else s


def quantize_with_scale(x: np.ndarray, s, fmt) -> np.ndarray:
    """Codes of x under a given fp32 scale: sat_rne(RN32(x / s))."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    q64 = x64 / np.asarray(s, dtype=np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        q32 = q64.astype(np.float32)
    # The quotient of finite x by a positive s is a finite real; where its fp32
    # rounding overflows it lies far beyond Vmax, so the code saturates
    # (reading G21) rather than becoming an E5M2 Inf.
    big = np.float32(np.finfo(np.float32).max)
    q32 = np.where(np.isinf(q32) & np.isfinite(q64), np.where(q64 < 0, -big, big), q32).astype(np.float32)
    return formats.encode(q32.astype(np.float64), fmt)


def quantize_delayed(x: np.ndarray, history: np.ndarray, pos: int, margin: int, fmt):
    """One iteration of delayed scaling on a tensor: the scale from the history
    as it stands, the codes under that scale (values beyond s*Vmax saturate),
    and the history with entry pos replaced by the tensor's amax.
    Returns (codes, s, new_history)."""
    s = delayed_scale(history, margin, fmt)
    codes = quantize_with_scale(x, s, fmt)
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.abs(x32).max()) if x32.size else np.float32(0.0)
    new_h = np.asarray(history, dtype=np.float32).copy()
    new_h[pos] = amax
    return codes, s, new_h



# ---- FP8 KV cache ------------------------------------------------------------
# "FP8 Mixed-Precision Serving", section "FP8 KV Cache Architecture and Serving
# Latency": key and value states stored as E4M3 codes (one byte per element,
# half of bf16), with the cache size 2 * B * L * N_heads * D_head * bytes per
# layer.  "FP8 Serving" (the quality table and "Things to try"): a per-tensor
# scale, a per-channel one for channel-structured outliers, and E5M2 as the
# format with more range.  The scales are static (given by the caller); the
# cache is a pool of token slots, each holding one token's [heads, head_dim]
# codes, addressed through a slot index per token (paged layouts map their
# block tables to slots).

KV_SCALE_TENSOR, KV_SCALE_HEAD, KV_SCALE_CHANNEL = 0, 1, 2


def kv_cache_bytes(batch: int, seq_len: int, heads: int, head_dim: int, bytes_per_element: int,
                   layers: int = 1) -> int:
    """Memory_KV = 2 * B * L * N_heads * D_head * BytesPerElement, times layers."""
    return 2 * batch * seq_len * heads * head_dim * bytes_per_element * layers


def kv_scale_of(scale_kind: int, scales, heads: int, head_dim: int) -> np.ndarray:
    """The fp32 scale of every element of a slot, [heads, head_dim]: one scale
    (per tensor), one per head, or one per channel (head, dim)."""
    s = np.asarray(scales, dtype=np.float32).reshape(-1)
    if scale_kind == KV_SCALE_TENSOR:
        return np.full((heads, head_dim), s[0], np.float32)
    if scale_kind == KV_SCALE_HEAD:
        return np.repeat(s[:heads, None], head_dim, axis=1).astype(np.float32)
    if scale_kind == KV_SCALE_CHANNEL:
        return s[:heads * head_dim].reshape(heads, head_dim).copy()
    raise ValueError(scale_kind)


def kv_append(cache: np.ndarray, x: np.ndarray, slots, scale_kind: int, scales, fmt) -> np.ndarray:
    """Quantize on append: token t of x [tokens, heads, head_dim] is written as
    codes sat_rne(RN32(x / s)) into cache[slots[t]]; a slot outside
    [0, num_slots) leaves the cache untouched (reading G22).  Returns a new
    cache [num_slots, heads, head_dim]."""
    out = np.array(cache, dtype=np.uint8, copy=True)
    slots = np.asarray(slots, dtype=np.int64)
    tokens, heads, head_dim = x.shape
    s = kv_scale_of(scale_kind, scales, heads, head_dim)
    for t in range(tokens):
        if 0 <= slots[t] < out.shape[0]:
            out[slots[t]] = quantize_with_scale(x[t], s, fmt)
    return out


def kv_gather(cache: np.ndarray, slots, scale_kind: int, scales, fmt) -> np.ndarray:
    """Dequantize on read: row i is RN32(decode(cache[slots[i]]) * s) as float32
    [n, heads, head_dim]; a slot outside [0, num_slots) reads as zeros
    (reading G22)."""
    cache = np.asarray(cache, dtype=np.uint8)
    num_slots, heads, head_dim = cache.shape
    slots = np.asarray(slots, dtype=np.int64)
    s = kv_scale_of(scale_kind, scales, heads, head_dim).astype(np.float64)
    out = np.zeros((len(slots), heads, head_dim), np.float32)
    for i, slot in enumerate(slots):
        if 0 <= slot < num_slots:
            v = formats.decode(cache[slot], fmt) * s
            with np.errstate(over="ignore", invalid="ignore"):
                out[i] = v.astype(np.float32)
    return out
