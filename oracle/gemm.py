"""Block-scaled FP8 GEMM reference and the elementwise tolerance (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The GEMM the path computes is Out = (X_fp8 * s_X) @ (W_fp8 * s_W)^T with an fp32
accumulator, i.e. s_X * s_W * (X_fp8 @ W_fp8^T) ("The FP8 Family", section
"Scaling is what makes FP8 usable", the MMA identity; "Illustrated GPU kernels,
Part 8", the paragraph before the qdq listing).  X is [M, K], W is [N, K], both
K-contiguous; Out is [M, N].  With per-128-K scales the same sum is taken block
by block, sum_kb s_X[m,kb] s_W[n,kb] P_kb ("The FP8 Family", DeepSeek-V3
callout, accumulator promotion; "Part 8", the promotion paragraph).

The reference is that product evaluated on the dequantized operands in fp64:
x_hat = decode(q_X) * s_X and w_hat = decode(q_W) * s_W are exact in fp64 (at
most 4 x 24 significant bits), Ref = x_hat @ w_hat^T, and the error bound's
scale is Abs = |x_hat| @ |w_hat|^T = sum_k |x_k w_k|.

Tolerance: |out - Ref| <= 1e-4 * Abs elementwise for fp32 outputs.  A bf16
output also carries its own final rounding, at most half a bf16 ulp of the
output, so it is held to 1e-4 * Abs + ulp_bf16(max(|out|, |Ref|)) / 2.
"""

from __future__ import annotations

import numpy as np

from . import formats, quant

REL_TOL = 1e-4


def dequant_operand(codes: np.ndarray, scales: np.ndarray, gran: int, fmt) -> np.ndarray:
    """Exact fp64 values of a quantized [rows, K] operand."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, cols = codes.shape
    return formats.decode(codes, fmt) * quant.broadcast_scale(scales, gran, rows, cols)


def dequant_rows(codes_rows: np.ndarray, scales: np.ndarray, gran: int, fmt,
                 row_ids: np.ndarray) -> np.ndarray:
    """Exact fp64 values of selected rows of a quantized operand.

    codes_rows: uint8 [len(row_ids), K], the codes of those rows;
    scales: the operand's full scale array."""
    codes_rows = np.asarray(codes_rows, dtype=np.uint8)
    row_ids = np.asarray(row_ids, dtype=np.int64)
    n, K = codes_rows.shape
    vals = formats.decode(codes_rows, fmt)
    if gran == quant.TENSOR:
        s = np.full((n, K), float(np.asarray(scales, np.float32).reshape(-1)[0]))
    elif gran == quant.ROW:
        s = np.repeat(np.asarray(scales, np.float32).reshape(-1)[row_ids].astype(np.float64)[:, None], K, axis=1)
    elif gran == quant.TILE_1x128:
        s = np.repeat(np.asarray(scales, np.float32).reshape(-1, K // 128)[row_ids].astype(np.float64), 128, axis=1)
    elif gran == quant.BLOCK_128x128:
        s = np.repeat(np.asarray(scales, np.float32).reshape(-1, K // 128)[row_ids // 128].astype(np.float64), 128, axis=1)
    elif gran == quant.MX32:
        b = np.asarray(scales, np.int64).reshape(-1, K // 32)[row_ids]
        s = np.repeat(np.where(b == 255, np.nan, np.ldexp(1.0, b - 127)), 32, axis=1)
    else:
        raise ValueError(gran)
    return vals * s


def gemm_ref(xq, sx, x_gran, x_fmt, wq, sw, w_gran, w_fmt):
    """(Ref, Abs), both fp64 [M, N]."""
    xh = dequant_operand(xq, sx, x_gran, x_fmt)
    wh = dequant_operand(wq, sw, w_gran, w_fmt)
    return xh @ wh.T, np.abs(xh) @ np.abs(wh).T


def gemm_ref_pairs(x_rows_hat: np.ndarray, w_rows_hat: np.ndarray, mi: np.ndarray, ni: np.ndarray):
    """Ref and Abs at output positions (mi[j], ni[j]) from dequantized row sets
    (x_rows_hat[i] is row mi-index i of x_hat, likewise for w)."""
    a = x_rows_hat[mi]
    b = w_rows_hat[ni]
    return np.einsum("ij,ij->i", a, b), np.einsum("ij,ij->i", np.abs(a), np.abs(b))


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (8 significant bits, min exponent -126)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, -126)
    return np.ldexp(1.0, e - 7)


def check_f32(out: np.ndarray, ref: np.ndarray, absb: np.ndarray, rel: float = REL_TOL):
    """Elementwise |out - Ref| <= rel * Abs.  Returns (ok_mask, worst_ratio)."""
    out = np.asarray(out, dtype=np.float64)
    err = np.abs(out - ref)
    bound = rel * absb
    ok = err <= bound
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    return ok, float(ratio.max()) if ratio.size else 0.0


def check_bf16(out_bits: np.ndarray, ref: np.ndarray, absb: np.ndarray, rel: float = REL_TOL):
    """Elementwise |out - Ref| <= rel * Abs + ulp_bf16(max(|out|,|Ref|)) / 2."""
    out = quant.bf16_bits_to_f64(out_bits)
    err = np.abs(out - ref)
    bound = rel * absb + 0.5 * ulp_bf16(np.maximum(np.abs(out), np.abs(ref)))
    ok = err <= bound
    ratio = err / bound
    return ok, float(ratio.max()) if ratio.size else 0.0
