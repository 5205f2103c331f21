"""Shared helpers of the GPU parity tests (host <-> device marshalling only)."""

import sys

import numpy as np
import torch

import workloads
from oracle import formats, gemm, quant


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype: int = None) -> torch.Tensor:
    """numpy -> device tensor.  uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def f32_of_store(a: np.ndarray) -> np.ndarray:
    return workloads.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a.astype(np.float32)


def oracle_quantize(x_store: np.ndarray, gran: int, fmt: int):
    return quant.quantize(f32_of_store(x_store), gran, fmt)


def assert_codes_equal(got: np.ndarray, want: np.ndarray, label: str, x=None):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (label, got.shape, want.shape)
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    if bad.size:
        i = bad[:8]
        extra = "" if x is None else f" inputs={np.asarray(x).reshape(-1)[i].tolist()}"
        raise AssertionError(f"{label}: {bad.size} mismatches; first at {i.tolist()}: "
                             f"got={got.reshape(-1)[i].tolist()} want={want.reshape(-1)[i].tolist()}{extra}")


def assert_scales_equal(got: np.ndarray, want: np.ndarray, label: str):
    g = np.asarray(got)
    w = np.asarray(want)
    if g.dtype == np.float32:
        g = g.view(np.uint32)
        w = np.asarray(w, np.float32).view(np.uint32)
    assert_codes_equal(g.reshape(w.shape), w, label + " scales")


# Bound for the FP8 instructions' own accumulation (accum=NATIVE): one group of
# 8 products can lose 7 * 2^-13 of its largest product, so 1e-3 * sum|x w|.
NATIVE_REL_TOL = 1e-3


def gemm_check(out: np.ndarray, out_dtype: int, ref: np.ndarray, absb: np.ndarray, label: str,
               rel: float = gemm.REL_TOL):
    if out_dtype == workloads.DT_F32:
        ok, worst = gemm.check_f32(out.astype(np.float64), ref, absb, rel)
    else:
        ok, worst = gemm.check_bf16(out, ref, absb, rel)
    if not ok.all():
        i = np.flatnonzero(~ok.reshape(-1))[:5]
        o = out.reshape(-1)[i]
        if out_dtype != workloads.DT_F32:
            o = quant.bf16_bits_to_f64(o)
        raise AssertionError(f"{label}: {(~ok).sum()} of {ok.size} outside tolerance (worst ratio {worst:.3g}); "
                             f"out={np.asarray(o).tolist()} ref={ref.reshape(-1)[i].tolist()} "
                             f"abs={absb.reshape(-1)[i].tolist()}")
    return worst


def decode_np(codes, fmt):
    return formats.decode(codes, fmt)


_FULL = {}


def full_operands(name: str):
    """Full-size workload operands and their oracle quantization (cached per
    session): (wl, x_store, w_store, xq, sx, wq, sw)."""
    if name not in _FULL:
        wl = workloads.CONFIGS[name]
        xs, ws = workloads.make_inputs(wl)
        xq, sx = oracle_quantize(xs, wl.x_gran, wl.x_fmt)
        wq, sw = oracle_quantize(ws, wl.w_gran, wl.w_fmt)
        _FULL.clear()          # keep one workload resident at a time
        _FULL[name] = (wl, xs, ws, xq, sx, wq, sw)
    return _FULL[name]
