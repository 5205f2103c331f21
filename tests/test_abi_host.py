"""The C-ABI library on the host: it loads, exports every function the header
declares, and rejects bad arguments with status codes before touching HIP
(so these run without a GPU)."""

import ctypes
import os
import re

import pytest

import block_scaled_precision_x128_amd as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8blk.h")
PROBE_HEADER = os.path.join(ROOT, "include", "fp8blk_probe.h")


def _ensure_built():
    if not os.path.exists(fb.LIB_PATH):
        from block_scaled_precision_x128_amd import build
        build.build()


def header_functions(path=HEADER, prefix=r"fp[48]_"):
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\**\s+\**(" + prefix + r"\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    _ensure_built()
    return fb.load_library()


def test_header_declares_the_binding_exports():
    assert header_functions() == sorted(fb.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    assert lib.fp8_abi_version() == 1


def test_probe_header_declares_the_binding_exports(lib):
    names = header_functions(PROBE_HEADER, r"fp8blk_probe_")
    assert names == sorted(fb.PROBE_EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_every_header_is_covered():
    # every header under include/ is one of the two checked above
    assert sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")) == \
        ["fp8blk.h", "fp8blk_probe.h"]


def test_probe_argument_checks(lib):
    flops = ctypes.c_double(0.0)
    assert lib.fp8blk_probe_mfma(7, 2, 1, FAKE, ctypes.byref(flops), None) == 2      # FP8_ERR_ENUM
    assert lib.fp8blk_probe_mfma(0, 3, 1, FAKE, ctypes.byref(flops), None) == 3      # FP8_ERR_SHAPE
    assert lib.fp8blk_probe_mfma(0, 2, 0, FAKE, ctypes.byref(flops), None) == 3
    assert lib.fp8blk_probe_mfma(0, 2, 1, None, ctypes.byref(flops), None) == 1      # FP8_ERR_NULL
    assert lib.fp8blk_probe_read(FAKE, 15, FAKE, None) == 3
    assert lib.fp8blk_probe_read(FAKE + 4, 16, FAKE, None) == 7                       # FP8_ERR_ALIGN
    assert lib.fp8blk_probe_copy(FAKE, FAKE + 64, 1024, None) == 3                     # overlapping
    assert lib.fp8blk_probe_copy(None, FAKE, 16, None) == 1
    assert lib.fp8blk_probe_read_sink_floats() == 1024 * 256
    assert lib.fp8blk_probe_mfma_sink_floats(3) == 0


def test_status_strings(lib):
    for st in range(8):
        assert lib.fp8_status_string(st)
    assert lib.fp8_status_string(99) == b"unknown status"


def test_workspace_query(lib):
    assert lib.fp8_quantize_workspace_bytes(128, 512, fb.GRAN_TENSOR) == 4 * 8192
    for g in (fb.GRAN_ROW, fb.GRAN_TILE_1x128, fb.GRAN_BLOCK_128x128, fb.GRAN_MX32):
        assert lib.fp8_quantize_workspace_bytes(128, 512, g) == 0
    assert lib.fp8_quantize_workspace_bytes(128, 500, fb.GRAN_TENSOR) == 0


FAKE = 1 << 20  # an aligned non-null address; never dereferenced by these calls


def test_quantize_validation(lib):
    q = lib.fp8_quantize
    assert q(FAKE, 0, 4, 128, 5, fb.GRAN_ROW, FAKE, FAKE, None, 0, None) == 2          # bad format
    assert q(FAKE, 7, 4, 128, 0, fb.GRAN_ROW, FAKE, FAKE, None, 0, None) == 2          # bad dtype
    assert q(FAKE, 0, 4, 128, 0, 9, FAKE, FAKE, None, 0, None) == 2                    # bad granularity
    assert q(FAKE, 0, 4, 100, 0, fb.GRAN_ROW, FAKE, FAKE, None, 0, None) == 3          # K % 128
    assert q(FAKE, 0, -1, 128, 0, fb.GRAN_ROW, FAKE, FAKE, None, 0, None) == 3         # negative
    assert q(FAKE, 0, 100, 128, 0, fb.GRAN_BLOCK_128x128, FAKE, FAKE, None, 0, None) == 3
    assert q(None, 0, 4, 128, 0, fb.GRAN_ROW, FAKE, FAKE, None, 0, None) == 1          # null x
    assert q(FAKE, 0, 4, 128, 0, fb.GRAN_ROW, FAKE, None, None, 0, None) == 1          # null scales
    assert q(FAKE + 8, 0, 4, 128, 0, fb.GRAN_ROW, FAKE, FAKE, None, 0, None) == 7      # misaligned x
    assert q(FAKE, 0, 4, 128, 0, fb.GRAN_ROW, FAKE, FAKE + 2, None, 0, None) == 7      # misaligned scales
    assert q(FAKE, 0, 4, 128, 0, fb.GRAN_TENSOR, FAKE, FAKE, None, 0, None) == 5       # no workspace
    assert q(FAKE, 0, 4, 128, 0, fb.GRAN_TENSOR, FAKE, FAKE, FAKE, 100, None) == 5     # small workspace
    assert q(FAKE, 0, 2 ** 62, 2 ** 20, 0, fb.GRAN_ROW, FAKE, FAKE, None, 0, None) == 3  # overflow
    # empty input with a non-tensor granularity is a no-op that needs no pointers
    assert q(None, 0, 0, 128, 0, fb.GRAN_ROW, None, None, None, 0, None) == 0


def test_dequantize_and_cast_validation(lib):
    d = lib.fp8_dequantize
    assert d(FAKE, FAKE, 4, 128, 3, 0, FAKE, 0, None) == 2
    assert d(FAKE, FAKE, 4, 120, 0, 0, FAKE, 0, None) == 3
    assert d(None, FAKE, 4, 128, 0, 0, FAKE, 0, None) == 1
    assert d(FAKE, FAKE, 4, 128, 0, 0, FAKE + 4, 0, None) == 7
    assert d(None, None, 0, 128, 0, 0, None, 0, None) == 0
    c = lib.fp8_cast
    assert c(FAKE, 0, 12, 0, FAKE, None) == 3
    assert c(FAKE, 0, 16, 2, FAKE, None) == 2
    assert c(None, 0, 16, 0, FAKE, None) == 1
    assert c(None, 0, 0, 0, None, None) == 0


def test_gemm_validation(lib):
    g = lib.fp8_gemm_blockscaled_ex
    T, R, TL, BL, MX = (fb.GRAN_TENSOR, fb.GRAN_ROW, fb.GRAN_TILE_1x128, fb.GRAN_BLOCK_128x128, fb.GRAN_MX32)
    args = lambda ag, bg, M=32, N=128, K=256, out=FAKE, algo=0, a=FAKE, od=1, acc=0: (
        a, 0, ag, FAKE, FAKE, 0, bg, FAKE, M, N, K, out, od, algo, acc, None)
    assert g(*args(TL, TL)) == 4             # unsupported pair
    assert g(*args(MX, T)) == 4
    assert g(*args(BL, BL)) == 4
    assert g(*args(T, T, M=24)) == 3         # M % 16
    assert g(*args(T, T, K=200)) == 3        # K % 128
    assert g(*args(T, T, K=(1 << 22) + 128)) == 3   # K beyond 32-bit buffer offsets
    assert g(*args(TL, BL, N=144)) == 3      # 128x128 blocks need N % 128
    assert g(*args(T, T, algo=5)) == 2
    assert g(*args(T, T, M=128, algo=fb.GEMM_SKINNY)) == 4
    assert g(*args(T, T, a=None)) == 1
    assert g(*args(T, T, out=None)) == 1
    assert g(*args(T, T, a=FAKE + 1)) == 7
    assert g(*args(T, T, od=3)) == 2
    assert g(*args(T, T, acc=2)) == 2
    assert g(*args(T, T, M=0)) == 0          # empty output: nothing to do


def test_gemm_quant_validation(lib):
    g = lib.fp8_gemm_blockscaled_quant
    T, TL, BL = fb.GRAN_TENSOR, fb.GRAN_TILE_1x128, fb.GRAN_BLOCK_128x128
    args = lambda ag, bg, M=32, N=256, K=256, fmt=0, codes=FAKE, scales=FAKE: (
        FAKE, 0, ag, FAKE, FAKE, 0, bg, FAKE, M, N, K, fmt, codes, scales, 0, None)
    assert g(*args(T, T, N=144)) == 3          # N % 128 for the 1x128 output tiles
    assert g(*args(T, T, fmt=2)) == 2          # output format
    assert g(*args(TL, TL)) == 4               # unsupported pair
    assert g(*args(T, T, codes=None)) == 1
    assert g(*args(T, T, scales=FAKE + 2)) == 7
    assert g(*args(T, T, codes=FAKE + 8)) == 7
    assert g(*args(TL, BL, M=0)) == 0          # empty output: nothing to do



def test_quantize_delayed_validation(lib):
    f = lib.fp8_quantize_delayed
    args = lambda rows=4, cols=128, fmt=0, hist=FAKE, hl=8, hp=0, m=0, q=FAKE, sc=FAKE, ws=FAKE, wsb=32768: (
        FAKE, 0, rows, cols, fmt, hist, hl, hp, m, q, sc, ws, wsb, None)
    assert f(*args(fmt=3)) == 2
    assert f(*args(cols=100)) == 3            # cols % 128
    assert f(*args(hp=8)) == 3                # position outside the history
    assert f(*args(hl=0)) == 3
    assert f(*args(m=32)) == 3                # margin outside 0..31
    assert f(*args(hist=None)) == 1
    assert f(*args(sc=None)) == 1
    assert f(*args(ws=None)) == 5
    assert f(*args(wsb=16)) == 5
    assert f(*args(sc=FAKE + 2)) == 7


def test_kv_append_validation(lib):
    f = lib.fp8_kv_append
    args = lambda x=FAKE, dt=1, t=4, h=8, d=128, ld=1024, sl=FAKE, fmt=0, sk=0, sc=FAKE, c=FAKE, ns=64: (
        x, dt, t, h, d, ld, sl, fmt, sk, sc, c, ns, None)
    assert f(*args(dt=2)) == 2
    assert f(*args(fmt=2)) == 2
    assert f(*args(sk=3)) == 2
    assert f(*args(d=120)) == 3               # head_dim % 16
    assert f(*args(h=-1)) == 3
    assert f(*args(ns=-1)) == 3
    assert f(*args(ld=1000)) == 3             # stride shorter than a row
    assert f(*args(h=1 << 20, d=1 << 10)) == 3  # row over 2^24 elements
    assert f(*args(t=1 << 62)) == 3           # x size overflows
    assert f(*args(x=None)) == 1
    assert f(*args(sl=None)) == 1
    assert f(*args(sc=None)) == 1
    assert f(*args(c=None)) == 1
    assert f(*args(ld=1028)) == 7             # bf16 rows not 16-byte aligned
    assert f(*args(x=FAKE + 8)) == 7
    assert f(*args(sl=FAKE + 4)) == 7
    assert f(*args(sc=FAKE + 2)) == 7
    assert f(*args(c=FAKE + 8)) == 7
    # nothing to do: no launch, OK even with null pointers
    assert f(*args(t=0, x=None, sl=None, c=None)) == 0
    assert f(*args(h=0, x=None, sl=None, c=None)) == 0


def test_kv_gather_validation(lib):
    f = lib.fp8_kv_gather
    args = lambda c=FAKE, ns=64, h=8, d=128, sl=FAKE, n=4, fmt=1, sk=2, sc=FAKE, o=FAKE, odt=1: (
        c, ns, h, d, sl, n, fmt, sk, sc, o, odt, None)
    assert f(*args(odt=5)) == 2
    assert f(*args(sk=-1)) == 2
    assert f(*args(d=8)) == 3
    assert f(*args(n=-2)) == 3
    assert f(*args(n=1 << 62)) == 3
    assert f(*args(sl=None)) == 1
    assert f(*args(sc=None)) == 1
    assert f(*args(o=None)) == 1
    assert f(*args(c=None)) == 1
    assert f(*args(o=FAKE + 4)) == 7
    assert f(*args(c=FAKE + 1)) == 7
    assert f(*args(n=0, sl=None, o=None)) == 0


def test_fp4_validation(lib):
    f = lib.fp4_quantize
    args = lambda x=FAKE, dt=1, rows=4, cols=256, kind=1, q=FAKE, bs=FAKE, ts=FAKE, ws=FAKE, wsb=32768: (
        x, dt, rows, cols, kind, q, bs, ts, ws, wsb, None)
    assert lib.fp4_quantize_workspace_bytes(4, 256, 1) == 32768
    assert lib.fp4_quantize_workspace_bytes(4, 256, 0) == 0
    assert lib.fp4_quantize_workspace_bytes(4, 250, 1) == 0
    assert f(*args(kind=2)) == 2
    assert f(*args(dt=3)) == 2
    assert f(*args(cols=200)) == 3
    assert f(*args(x=None)) == 1
    assert f(*args(bs=None)) == 1
    assert f(*args(ts=None)) == 1            # NV needs the tensor scale
    assert f(*args(ws=None)) == 5
    assert f(*args(wsb=100)) == 5
    assert f(*args(q=FAKE + 4)) == 7
    assert f(*args(ts=FAKE + 1)) == 7
    assert f(*args(kind=0, ts=None, ws=None, wsb=0, rows=0)) == 0   # empty MX: nothing to do
    d = lib.fp4_dequantize
    dargs = lambda q=FAKE, bs=FAKE, ts=FAKE, rows=4, cols=256, kind=1, y=FAKE, dt=0: (q, bs, ts, rows, cols, kind, y, dt, None)
    assert d(*dargs(kind=5)) == 2
    assert d(*dargs(cols=100)) == 3
    assert d(*dargs(ts=None)) == 1
    assert d(*dargs(y=FAKE + 8)) == 7
    assert d(*dargs(rows=0, q=None, y=None)) == 0


def test_library_exports_nothing_else(lib):
    """The C symbols the library exports are exactly the headers' functions."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", fb.LIB_PATH], capture_output=True, text=True, check=True).stdout
    c_syms = sorted(l.split()[-1] for l in out.splitlines() if " T " in l and not l.split()[-1].startswith("_Z"))
    assert c_syms == sorted(header_functions() + header_functions(PROBE_HEADER, r"fp8blk_probe_"))


def test_fp4_gemm_validation(lib):
    f = lib.fp4_gemm_blockscaled
    args = lambda a=FAKE, sa=FAKE, ta=FAKE, b=FAKE, sb=FAKE, tb=FAKE, M=32, N=32, K=512, kind=1, out=FAKE, odt=0: (
        a, sa, ta, b, sb, tb, M, N, K, kind, out, odt, None)
    assert f(*args(kind=2)) == 2
    assert f(*args(odt=2)) == 2
    assert f(*args(K=384)) == 3               # K % 256
    assert f(*args(M=24)) == 3
    assert f(*args(K=1 << 23)) == 3
    assert f(*args(ta=None)) == 1             # NV needs the tensor scales
    assert f(*args(sb=None)) == 1
    assert f(*args(out=None)) == 1
    assert f(*args(a=FAKE + 8)) == 7
    assert f(*args(sa=FAKE + 2)) == 7
    assert f(*args(kind=0, ta=None, tb=None, a=FAKE + 8)) == 7   # MX ignores the tensor scales
    assert f(*args(M=0, a=None, out=None)) == 0
