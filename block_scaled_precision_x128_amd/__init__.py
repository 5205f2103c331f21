"""Python binding of libfp8blk, the MI355X (gfx950) FP8 quantize + block-scaled
FP8 GEMM library.

The functions mirror the C ABI in include/fp8blk.h by name.  They only marshal
arguments: torch tensors supply device memory and the current HIP stream, every
step of the computation runs in the library's HIP kernels.  When the library
is missing or no GPU is present, every call raises; there is no CPU fallback.

Enum values (same as the C header):
  formats        E4M3 = 0, E5M2 = 1
  granularities  GRAN_TENSOR = 0, GRAN_ROW = 1, GRAN_TILE_1x128 = 2,
                 GRAN_BLOCK_128x128 = 3, GRAN_MX32 = 4
  dtypes         DT_F32 = 0, DT_BF16 = 1
  GEMM kernels   GEMM_AUTO = 0, GEMM_TILED = 1, GEMM_SKINNY = 2
  accumulation   ACCUM_FP32 = 0 (exact products, fp32 sums), ACCUM_NATIVE = 1
  KV scales      KV_SCALE_TENSOR = 0, KV_SCALE_HEAD = 1, KV_SCALE_CHANNEL = 2
  FP4 scaling    FP4_MX = 0 (32-element UE8M0), FP4_NV = 1 (16-element E4M3 + fp32 tensor)
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

E4M3, E5M2 = 0, 1
GRAN_TENSOR, GRAN_ROW, GRAN_TILE_1x128, GRAN_BLOCK_128x128, GRAN_MX32 = 0, 1, 2, 3, 4
DT_F32, DT_BF16 = 0, 1
GEMM_AUTO, GEMM_TILED, GEMM_SKINNY = 0, 1, 2
ACCUM_FP32, ACCUM_NATIVE = 0, 1
KV_SCALE_TENSOR, KV_SCALE_HEAD, KV_SCALE_CHANNEL = 0, 1, 2
FP4_MX, FP4_NV = 0, 1

FP8_OK = 0
STATUS_NAMES = {0: "FP8_OK", 1: "FP8_ERR_NULL", 2: "FP8_ERR_ENUM", 3: "FP8_ERR_SHAPE",
                4: "FP8_ERR_UNSUPPORTED", 5: "FP8_ERR_WORKSPACE", 6: "FP8_ERR_HIP", 7: "FP8_ERR_ALIGN"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8blk.so")

# Exported symbols and their C signatures (include/fp8blk.h).
_c = ctypes
_SIGS = {
    "fp8_status_string": (_c.c_char_p, [_c.c_int]),
    "fp8_abi_version": (_c.c_int, []),
    "fp8_quantize_workspace_bytes": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int]),
    "fp8_quantize": (_c.c_int, [_c.c_void_p, _c.c_int, _c.c_int64, _c.c_int64, _c.c_int, _c.c_int,
                                _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "fp8_quantize_noalloc": (_c.c_int, [_c.c_void_p, _c.c_int, _c.c_int64, _c.c_int64, _c.c_int, _c.c_int,
                                        _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "fp8_quantize_delayed": (_c.c_int, [_c.c_void_p, _c.c_int, _c.c_int64, _c.c_int64, _c.c_int, _c.c_void_p,
                                        _c.c_int64, _c.c_int64, _c.c_int, _c.c_void_p, _c.c_void_p,
                                        _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "fp8_dequantize": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int, _c.c_int,
                                  _c.c_void_p, _c.c_int, _c.c_void_p]),
    "fp8_cast": (_c.c_int, [_c.c_void_p, _c.c_int, _c.c_int64, _c.c_int, _c.c_void_p, _c.c_void_p]),
    "fp8_gemm_blockscaled": (_c.c_int, [_c.c_void_p, _c.c_int, _c.c_int, _c.c_void_p,
                                        _c.c_void_p, _c.c_int, _c.c_int, _c.c_void_p,
                                        _c.c_int64, _c.c_int64, _c.c_int64,
                                        _c.c_void_p, _c.c_int, _c.c_void_p]),
    "fp8_gemm_blockscaled_ex": (_c.c_int, [_c.c_void_p, _c.c_int, _c.c_int, _c.c_void_p,
                                           _c.c_void_p, _c.c_int, _c.c_int, _c.c_void_p,
                                           _c.c_int64, _c.c_int64, _c.c_int64,
                                           _c.c_void_p, _c.c_int, _c.c_int, _c.c_int, _c.c_void_p]),
    "fp8_gemm_blockscaled_quant": (_c.c_int, [_c.c_void_p, _c.c_int, _c.c_int, _c.c_void_p,
                                              _c.c_void_p, _c.c_int, _c.c_int, _c.c_void_p,
                                              _c.c_int64, _c.c_int64, _c.c_int64,
                                              _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_void_p]),
    "fp8_kv_append": (_c.c_int, [_c.c_void_p, _c.c_int, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int64,
                                 _c.c_void_p, _c.c_int, _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_int64,
                                 _c.c_void_p]),
    "fp8_kv_gather": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_void_p, _c.c_int64,
                                 _c.c_int, _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_void_p]),
    "fp4_quantize_workspace_bytes": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int]),
    "fp4_quantize": (_c.c_int, [_c.c_void_p, _c.c_int, _c.c_int64, _c.c_int64, _c.c_int, _c.c_void_p,
                                _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "fp4_dequantize": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int,
                                  _c.c_void_p, _c.c_int, _c.c_void_p]),
    "fp4_gemm_blockscaled": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                        _c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_int, _c.c_void_p,
                                        _c.c_int, _c.c_void_p]),
}
EXPORTS = tuple(_SIGS)

# Measurement probes (include/fp8blk_probe.h): not part of the method; they
# measure the machine's matrix-core, read and copy ceilings.
PROBE_MFMA_BF16, PROBE_MFMA_FP8 = 0, 1
_PROBE_SIGS = {
    "fp8blk_probe_mfma_sink_floats": (_c.c_size_t, [_c.c_int]),
    "fp8blk_probe_mfma": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_void_p, _c.POINTER(_c.c_double),
                                     _c.c_void_p]),
    "fp8blk_probe_read_sink_floats": (_c.c_size_t, []),
    "fp8blk_probe_read": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_void_p, _c.c_void_p]),
    "fp8blk_probe_copy": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_void_p]),
}
PROBE_EXPORTS = tuple(_PROBE_SIGS)

_lib: Optional[ctypes.CDLL] = None


class Fp8Error(RuntimeError):
    """A libfp8blk call returned a non-OK status."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} ({msg})")
        self.status = status


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libfp8blk.so (built by build.py) and declare its signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libfp8blk.so not found at {p}: build it with "
                           "`python -m block_scaled_precision_x128_amd.build` (there is no fallback)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in list(_SIGS.items()) + list(_PROBE_SIGS.items()):
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(fn: str, st: int):
    if st != FP8_OK:
        raise Fp8Error(fn, st, load_library().fp8_status_string(st).decode())


def _torch():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("libfp8blk needs a ROCm GPU; torch.cuda.is_available() is False")
    return torch


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _dt_of(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return DT_F32
    if t.dtype == torch.bfloat16:
        return DT_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _torch_dtype(dt: int):
    torch = _torch()
    return torch.float32 if dt == DT_F32 else torch.bfloat16


def scale_shape(gran: int, rows: int, cols: int):
    return {GRAN_TENSOR: (1,), GRAN_ROW: (rows,), GRAN_TILE_1x128: (rows, cols // 128),
            GRAN_BLOCK_128x128: (rows // 128, cols // 128), GRAN_MX32: (rows, cols // 32)}[gran]


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


# ---- raw entry points (pointers and sizes, as in C) -------------------------

def fp8_status_string(status: int) -> str:
    return load_library().fp8_status_string(status).decode()


def fp8_abi_version() -> int:
    return load_library().fp8_abi_version()


def fp8_quantize_workspace_bytes(rows: int, cols: int, gran: int) -> int:
    return load_library().fp8_quantize_workspace_bytes(rows, cols, gran)


# ---- tensor-level wrappers ----------------------------------------------------

def fp8_quantize(x, fmt: int, gran: int, q=None, scales=None, workspace=None, stream=None):
    """Quantize a 2-D fp32/bf16 device tensor.  Returns (codes uint8, scales)."""
    torch = _torch()
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scales is None:
        sdt = torch.uint8 if gran == GRAN_MX32 else torch.float32
        scales = torch.empty(scale_shape(gran, rows, cols), dtype=sdt, device=x.device)
    lib = load_library()
    ws = lib.fp8_quantize_workspace_bytes(rows, cols, gran)
    if ws and workspace is None:
        workspace = torch.empty(ws, dtype=torch.uint8, device=x.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.fp8_quantize(x.data_ptr(), _dt_of(x), rows, cols, fmt, gran, q.data_ptr(), scales.data_ptr(),
                          _ptr(workspace), wsb, _stream(stream))
    _check("fp8_quantize", st)
    return q, scales


def fp8_quantize_noalloc(x, fmt: int, gran: int, q, scales, stream=None):
    """fp8_quantize into caller-provided q and scales with no workspace: the
    per-tensor amax partials live in the library's static device scratch
    (calls that overlap on one GPU race).  Returns (q, scales)."""
    rows, cols = x.shape
    st = load_library().fp8_quantize_noalloc(x.data_ptr(), _dt_of(x), rows, cols, fmt, gran, q.data_ptr(),
                                             scales.data_ptr(), _stream(stream))
    _check("fp8_quantize_noalloc", st)
    return q, scales


def fp8_quantize_delayed(x, fmt: int, history, hist_pos: int, margin: int = 0, q=None, scale=None, workspace=None,
                         stream=None):
    """Delayed scaling: quantize x (2-D) with the scale from the amax history
    (device float32 [l]), then store x's amax at history[hist_pos].
    Returns (codes uint8, scale float32 [1])."""
    torch = _torch()
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    lib = load_library()
    ws = lib.fp8_quantize_workspace_bytes(rows, cols, GRAN_TENSOR)
    if ws and workspace is None:
        workspace = torch.empty(ws, dtype=torch.uint8, device=x.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.fp8_quantize_delayed(x.data_ptr(), _dt_of(x), rows, cols, fmt, history.data_ptr(), history.numel(),
                                  hist_pos, margin, q.data_ptr(), scale.data_ptr(), _ptr(workspace), wsb,
                                  _stream(stream))
    _check("fp8_quantize_delayed", st)
    return q, scale


def fp8_dequantize(q, scales, fmt: int, gran: int, out_dtype: int = DT_F32, y=None, stream=None):
    """Dequantize codes to fp32 or bf16.  Returns y."""
    torch = _torch()
    rows, cols = q.shape
    if y is None:
        y = torch.empty((rows, cols), dtype=_torch_dtype(out_dtype), device=q.device)
    st = load_library().fp8_dequantize(q.data_ptr(), scales.data_ptr(), rows, cols, fmt, gran, y.data_ptr(),
                                       out_dtype, _stream(stream))
    _check("fp8_dequantize", st)
    return y


def fp8_cast(x, fmt: int, q=None, stream=None):
    """Unscaled saturating cast of a fp32/bf16 device tensor (numel % 8 == 0)."""
    torch = _torch()
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    st = load_library().fp8_cast(x.data_ptr(), _dt_of(x), x.numel(), fmt, q.data_ptr(), _stream(stream))
    _check("fp8_cast", st)
    return q


def fp8_gemm_blockscaled(a, a_fmt: int, a_gran: int, a_scales, b, b_fmt: int, b_gran: int, b_scales,
                         out_dtype: int = DT_BF16, out=None, algo: int = GEMM_AUTO, accum: int = ACCUM_FP32,
                         stream=None):
    """out[M, N] = (a * sA) @ (b * sB)^T for codes a [M, K], b [N, K]."""
    torch = _torch()
    M, K = a.shape
    N = b.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=_torch_dtype(out_dtype), device=a.device)
    lib = load_library()
    if algo == GEMM_AUTO and accum == ACCUM_FP32:
        # the plain entry point (AUTO kernel choice, exact products with fp32 sums)
        st = lib.fp8_gemm_blockscaled(
            a.data_ptr(), a_fmt, a_gran, a_scales.data_ptr(), b.data_ptr(), b_fmt, b_gran, b_scales.data_ptr(),
            M, N, K, out.data_ptr(), out_dtype, _stream(stream))
    else:
        st = lib.fp8_gemm_blockscaled_ex(
            a.data_ptr(), a_fmt, a_gran, a_scales.data_ptr(), b.data_ptr(), b_fmt, b_gran, b_scales.data_ptr(),
            M, N, K, out.data_ptr(), out_dtype, algo, accum, _stream(stream))
    _check("fp8_gemm_blockscaled", st)
    return out


def fp8_gemm_blockscaled_quant(a, a_fmt: int, a_gran: int, a_scales, b, b_fmt: int, b_gran: int, b_scales,
                               out_fmt: int = E4M3, codes=None, scales=None, accum: int = ACCUM_FP32, stream=None):
    """The GEMM with its result quantized in the epilogue to out_fmt codes and
    1x128 tile scales (the layout fp8_quantize writes for GRAN_TILE_1x128).
    Returns (codes uint8 [M, N], scales float32 [M, N/128])."""
    torch = _torch()
    M, K = a.shape
    N = b.shape[0]
    if codes is None:
        codes = torch.empty((M, N), dtype=torch.uint8, device=a.device)
    if scales is None:
        scales = torch.empty((M, N // 128), dtype=torch.float32, device=a.device)
    st = load_library().fp8_gemm_blockscaled_quant(
        a.data_ptr(), a_fmt, a_gran, a_scales.data_ptr(), b.data_ptr(), b_fmt, b_gran, b_scales.data_ptr(),
        M, N, K, out_fmt, codes.data_ptr(), scales.data_ptr(), accum, _stream(stream))
    _check("fp8_gemm_blockscaled_quant", st)
    return codes, scales


def fp8_kv_append(x, slots, cache, scales, fmt: int, scale_kind: int, stream=None):
    """Quantize on append: x [tokens, heads, head_dim] (fp32 or bf16; the
    leading dimension may be strided, e.g. a slice of a fused QKV output)
    written as codes into cache [num_slots, heads, head_dim] at rows slots
    (int64 [tokens]; slots outside the pool are skipped).  Returns cache."""
    tokens, heads, head_dim = x.shape
    if x.stride(2) != 1 or x.stride(1) != head_dim:
        raise ValueError("x must be contiguous within a token ([heads, head_dim] row-major)")
    if tuple(cache.shape[1:]) != (heads, head_dim) or not cache.is_contiguous():
        raise ValueError("cache must be a contiguous [num_slots, heads, head_dim] uint8 tensor")
    st = load_library().fp8_kv_append(x.data_ptr(), _dt_of(x), tokens, heads, head_dim, x.stride(0),
                                      slots.data_ptr(), fmt, scale_kind, scales.data_ptr(), cache.data_ptr(),
                                      cache.shape[0], _stream(stream))
    _check("fp8_kv_append", st)
    return cache


def fp8_kv_gather(cache, slots, scales, fmt: int, scale_kind: int, out_dtype: int = DT_BF16, out=None,
                  stream=None):
    """Dequantize on read: rows slots (int64 [n]) of cache [num_slots, heads,
    head_dim] as fp32 or bf16 [n, heads, head_dim] (zeros for slots outside the
    pool).  Returns out."""
    torch = _torch()
    num_slots, heads, head_dim = cache.shape
    n = slots.shape[0]
    if out is None:
        out = torch.empty((n, heads, head_dim), dtype=_torch_dtype(out_dtype), device=cache.device)
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    st = load_library().fp8_kv_gather(cache.data_ptr(), num_slots, heads, head_dim, slots.data_ptr(), n, fmt,
                                      scale_kind, scales.data_ptr(), out.data_ptr(), _dt_of(out), _stream(stream))
    _check("fp8_kv_gather", st)
    return out


def fp4_block(kind: int) -> int:
    return 32 if kind == FP4_MX else 16


def fp4_quantize_workspace_bytes(rows: int, cols: int, kind: int) -> int:
    return int(load_library().fp4_quantize_workspace_bytes(rows, cols, kind))


def fp4_quantize(x, kind: int, q=None, block_scales=None, tensor_scale=None, workspace=None, stream=None):
    """Quantize x [rows, cols] to packed E2M1 codes.  Returns (q [rows, cols/2]
    uint8, block_scales uint8 [rows, cols/32 or cols/16], tensor_scale float32
    [1] or None for MX)."""
    torch = _torch()
    rows, cols = x.shape
    dev = x.device
    if q is None:
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    if block_scales is None:
        block_scales = torch.empty((rows, cols // fp4_block(kind)), dtype=torch.uint8, device=dev)
    if kind == FP4_NV and tensor_scale is None:
        tensor_scale = torch.empty(1, dtype=torch.float32, device=dev)
    wsb = fp4_quantize_workspace_bytes(rows, cols, kind)
    if workspace is None and wsb:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    st = load_library().fp4_quantize(x.data_ptr(), _dt_of(x), rows, cols, kind, q.data_ptr(),
                                     block_scales.data_ptr(), _ptr(tensor_scale), _ptr(workspace),
                                     workspace.numel() if workspace is not None else 0, _stream(stream))
    _check("fp4_quantize", st)
    return q, block_scales, tensor_scale


def fp4_dequantize(q, block_scales, tensor_scale, kind: int, out_dtype: int = DT_F32, y=None, stream=None):
    """Dequantize packed E2M1 codes [rows, cols/2] to fp32 or bf16 [rows, cols]."""
    torch = _torch()
    rows, half = q.shape
    if y is None:
        y = torch.empty((rows, 2 * half), dtype=_torch_dtype(out_dtype), device=q.device)
    st = load_library().fp4_dequantize(q.data_ptr(), block_scales.data_ptr(), _ptr(tensor_scale), rows, 2 * half,
                                       kind, y.data_ptr(), _dt_of(y), _stream(stream))
    _check("fp4_dequantize", st)
    return y


def fp4_gemm_blockscaled(a, a_scales, a_tensor_scale, b, b_scales, b_tensor_scale, kind: int,
                         out_dtype: int = DT_F32, out=None, stream=None):
    """FP4 block-scaled GEMM of packed E2M1 operands a [M, K/2], b [N, K/2]
    (K-contiguous) with their block (and, NV, tensor) scales.  MXFP4 runs on
    the FP4 matrix cores, NVFP4 on exact fp16 expansions; M <= 64 takes the
    skinny (decode) kernel.  Returns out [M, N]."""
    torch = _torch()
    M, half = a.shape
    N = b.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=_torch_dtype(out_dtype), device=a.device)
    st = load_library().fp4_gemm_blockscaled(a.data_ptr(), a_scales.data_ptr(), _ptr(a_tensor_scale), b.data_ptr(),
                                             b_scales.data_ptr(), _ptr(b_tensor_scale), M, N, 2 * half, kind,
                                             out.data_ptr(), _dt_of(out), _stream(stream))
    _check("fp4_gemm_blockscaled", st)
    return out


# ---- measurement probes (include/fp8blk_probe.h) -------------------------------

def probe_mfma(kind: int, waves_per_simd: int, iters: int, sink=None, stream=None) -> float:
    """Enqueue the back-to-back MFMA probe; returns the launch's FLOP count."""
    torch = _torch()
    lib = load_library()
    if sink is None:
        sink = torch.empty(int(lib.fp8blk_probe_mfma_sink_floats(waves_per_simd)), dtype=torch.float32,
                           device="cuda")
    flops = ctypes.c_double(0.0)
    st = lib.fp8blk_probe_mfma(kind, waves_per_simd, iters, sink.data_ptr(), ctypes.byref(flops), _stream(stream))
    _check("fp8blk_probe_mfma", st)
    return flops.value


def probe_read(src, sink=None, stream=None):
    """Enqueue a streaming read of every byte of the device tensor src."""
    torch = _torch()
    lib = load_library()
    if sink is None:
        sink = torch.empty(int(lib.fp8blk_probe_read_sink_floats()), dtype=torch.float32, device=src.device)
    st = lib.fp8blk_probe_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(), _stream(stream))
    _check("fp8blk_probe_read", st)
    return sink


def probe_copy(src, dst, stream=None):
    """Enqueue a device copy of src into dst (same byte size, no overlap)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same byte size")
    st = load_library().fp8blk_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream(stream))
    _check("fp8blk_probe_copy", st)
    return dst
