"""GPU parity: FP4 (E2M1) block-scaled GEMM, MXFP4 and NVFP4, against the
oracle's fp64 reference.  Operands are quantized by the oracle on the CPU and
the same codes and scales go to both sides.  Bound: |out - Ref| <= 1e-4 *
sum_k |deq(a) deq(b)| per element, plus half a bf16 ulp for bf16 outputs.

Shapes cover the three tile configurations: small problems (128x256 tiles),
4096x4096 (256x256) and 4096x4480 (256x256 plus a 256x192 column remainder),
with ragged M and N."""

import numpy as np
import pytest
import torch

import block_scaled_precision_x128_amd as fb
import workloads
from oracle import fp4
from gpu_helpers import dev, gemm_check, host, say

pytestmark = pytest.mark.gpu

KINDS = [fb.FP4_MX, fb.FP4_NV]


def _operands(kind, M, N, K, seed, wide=False):
    rng = np.random.default_rng(seed)
    wl = workloads.CONFIGS["c3_deepseek_block"]
    x = workloads.draw_x(wl, M, K, rng)
    w = workloads.draw_w(wl, N, K, rng)
    if wide:   # rows spanning many binades: the block scales differ widely along K
        x = (x * np.exp(rng.uniform(-8, 8, (1, K))).astype(np.float32)).astype(np.float32)
    if kind == fb.FP4_MX:
        a, sa = fp4.quantize_mx(x)
        b, sb = fp4.quantize_mx(w)
        return a, sa, None, b, sb, None
    a, sa, ta = fp4.quantize_nv(x)
    b, sb, tb = fp4.quantize_nv(w)
    return a, sa, np.array([ta], np.float32), b, sb, np.array([tb], np.float32)


def _run(kind, ops, out_dt):
    a, sa, ta, b, sb, tb = ops
    out = fb.fp4_gemm_blockscaled(dev(a), dev(sa), None if ta is None else dev(ta), dev(b), dev(sb),
                                  None if tb is None else dev(tb), kind, out_dt)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("out_dt", [fb.DT_F32, fb.DT_BF16])
@pytest.mark.parametrize("shape", [(16, 16, 256), (48, 80, 512), (272, 528, 768), (512, 1024, 2048),
                                   (400, 784, 1536)])
def test_fp4_gemm_small(kind, out_dt, shape):
    M, N, K = shape
    label = f"fp4 gemm kind={kind} out={out_dt} shape={shape}"
    say(label)
    ops = _operands(kind, M, N, K, 900 + kind + M + N)
    out = _run(kind, ops, out_dt)
    ref, absb = fp4.gemm_ref(kind, ops[0], ops[1], ops[3], ops[4], ops[2], ops[5])
    gemm_check(out, out_dt, ref, absb, label)


@pytest.mark.parametrize("kind", KINDS)
def test_fp4_gemm_wide_scales(kind):
    label = f"fp4 gemm wide scales kind={kind}"
    say(label)
    ops = _operands(kind, 64, 128, 1024, 950 + kind, wide=True)
    out = _run(kind, ops, fb.DT_F32)
    ref, absb = fp4.gemm_ref(kind, ops[0], ops[1], ops[3], ops[4], ops[2], ops[5])
    gemm_check(out, fb.DT_F32, ref, absb, label)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("N", [4096, 4480])
def test_fp4_gemm_large_tiles(kind, N):
    """4096 x N x 256: 256x256 tiles (N = 4096) and, with N = 4480, a ragged
    last tile column (NVFP4: the column split); every output is checked."""
    M, K = 4096, 256
    label = f"fp4 gemm large kind={kind} shape={(M, N, K)}"
    say(label)
    ops = _operands(kind, M, N, K, 970 + kind + N)
    out = _run(kind, ops, fb.DT_BF16)
    ref, absb = fp4.gemm_ref(kind, ops[0], ops[1], ops[3], ops[4], ops[2], ops[5])
    gemm_check(out, fb.DT_BF16, ref, absb, label)


@pytest.mark.parametrize("K", [1024, 1280])
def test_mxfp4_gemm_large_tiles_even_odd_steps(K):
    """MXFP4 at 4096 x 4352 x K on 256x256 tiles: K = 1024 has an even number
    of 256-K steps (two steps' scale bytes staged per load), K = 1280 an odd
    one (word-by-word staging); every output is checked."""
    M, N = 4096, 4352
    label = f"mxfp4 gemm large shape={(M, N, K)}"
    say(label)
    ops = _operands(fb.FP4_MX, M, N, K, 990 + K)
    out = _run(fb.FP4_MX, ops, fb.DT_BF16)
    ref, absb = fp4.gemm_ref(fb.FP4_MX, ops[0], ops[1], ops[3], ops[4], ops[2], ops[5])
    gemm_check(out, fb.DT_BF16, ref, absb, label)


def test_fp4_gemm_k_zero():
    say("fp4 gemm K=0")
    a = torch.zeros((32, 0), dtype=torch.uint8, device="cuda")
    s = torch.zeros((32, 0), dtype=torch.uint8, device="cuda")
    out = torch.full((32, 48), 7.0, device="cuda")
    b = torch.zeros((48, 0), dtype=torch.uint8, device="cuda")
    fb.fp4_gemm_blockscaled(a, s, None, b, s[:0], None, fb.FP4_MX, fb.DT_F32, out=out)
    torch.cuda.synchronize()
    assert not host(out).any()


@pytest.mark.parametrize("out_dt", [fb.DT_F32, fb.DT_BF16])
@pytest.mark.parametrize("shape", [(16, 18432, 1024), (48, 784, 2048), (64, 5008, 1536),
                                   (16, 48, 7168), (32, 784, 1536), (16, 528, 768), (32, 400, 1280)])
def test_mxfp4_gemm_decode_shapes(out_dt, shape):
    """MXFP4 with M <= 64 runs the skinny kernel on the FP4 matrix cores:
    workgroups own ceil(N / grid) weight rows (72 at N = 18432, not a whole
    number of 16-row tiles; 20 at N = 5008), the waves split K (ranges that
    start on odd steps included), and X rows past M read zeros.  M <= 32 with
    K % 512 == 0 stages the scale bytes of step pairs, the other shapes word
    by word.  Every output is checked."""
    M, N, K = shape
    label = f"mxfp4 decode gemm out={out_dt} shape={shape}"
    say(label)
    ops = _operands(fb.FP4_MX, M, N, K, 1700 + M + N + K)
    out = _run(fb.FP4_MX, ops, out_dt)
    ref, absb = fp4.gemm_ref(fb.FP4_MX, ops[0], ops[1], ops[3], ops[4], ops[2], ops[5])
    gemm_check(out, out_dt, ref, absb, label)


@pytest.mark.parametrize("out_dt", [fb.DT_F32, fb.DT_BF16])
@pytest.mark.parametrize("shape", [(16, 18432, 1024), (32, 784, 2048), (64, 5008, 1536), (48, 48, 7168)])
def test_nvfp4_gemm_decode_shapes(out_dt, shape):
    """NVFP4 with M <= 64 runs the skinny kernel on exact fp16 expansions:
    four microscale words per row and step, one to four X tiles (four column
    tiles per workgroup when M > 32), the tensor scales in the epilogue.
    Every output is checked."""
    M, N, K = shape
    label = f"nvfp4 decode gemm out={out_dt} shape={shape}"
    say(label)
    ops = _operands(fb.FP4_NV, M, N, K, 2700 + M + N + K)
    out = _run(fb.FP4_NV, ops, out_dt)
    ref, absb = fp4.gemm_ref(fb.FP4_NV, ops[0], ops[1], ops[3], ops[4], ops[2], ops[5])
    gemm_check(out, out_dt, ref, absb, label)


def _crafted_mx(rows, K, rng):
    """E2M1 codes (two per byte, element 2i in the low nibble) whose 32-element
    blocks each hold one +-6 among +-0.5s, or a +-6 that a -+6 cancels, and
    UE8M0 scales spread over 2^-25 .. 2^25."""
    codes = np.where(rng.random((rows, K)) < 0.5, 0x1, 0x9).astype(np.uint8)     # +-0.5
    blk = codes.reshape(rows, K // 32, 32)
    blk[:, :, 0] = np.where(rng.random((rows, K // 32)) < 0.5, 0x7, 0xF)          # +-6
    cancel = rng.random((rows, K // 32)) < 0.3
    blk[:, :, 1] = np.where(cancel, blk[:, :, 0] ^ 0x8, blk[:, :, 1])             # -+6 in some blocks
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(127 - 25, 127 + 26, (rows, K // 32)).astype(np.uint8)
    return packed, scales


@pytest.mark.parametrize("M", [16, 128])
def test_mxfp4_gemm_block_sums_exact(M):
    """The FP4 matrix cores on the widest in-block mix of E2M1 products (36
    against 0.25, and +-36 cancelling) with block scales over 2^-25 .. 2^25:
    every E2M1 block sum spans at most 13 bits, so it is formed exactly, and
    the scaled block sums and the K/128 instruction results are added in fp32.
    The result must stay within 1e-5 sum_k |x w|, ten times inside the
    contract's 1e-4 and above the worst case of those fp32 additions at
    K = 2048.  M = 16 runs the skinny kernel, M = 128 the tiled one."""
    rng = np.random.default_rng(4242 + M)
    N, K = 256, 2048
    a, sa = _crafted_mx(M, K, rng)
    b, sb = _crafted_mx(N, K, rng)
    label = f"mxfp4 crafted blocks M={M}"
    say(label)
    out = _run(fb.FP4_MX, (a, sa, None, b, sb, None), fb.DT_F32)
    ref, absb = fp4.gemm_ref(fb.FP4_MX, a, sa, b, sb)
    gemm_check(out, fb.DT_F32, ref, absb, label, rel=1e-5)


def _crafted_nv(rows, K, rng):
    """NVFP4 operands: E2M1 codes with one +-6 among +-0.5s per 16-element
    block (a -+6 cancelling it in some blocks), and E4M3 microscales drawn over
    E4M3's whole finite range (subnormal 2^-9 .. 448), so that one matrix-core
    instruction, which takes 8 elements from each of four blocks, holds
    products from 0.5 * 2^-9 * 0.5 * 2^-9 up to 2688 * 2688."""
    codes = np.where(rng.random((rows, K)) < 0.5, 0x1, 0x9).astype(np.uint8)
    blk = codes.reshape(rows, K // 16, 16)
    blk[:, :, 0] = np.where(rng.random((rows, K // 16)) < 0.5, 0x7, 0xF)
    cancel = rng.random((rows, K // 16)) < 0.3
    blk[:, :, 1] = np.where(cancel, blk[:, :, 0] ^ 0x8, blk[:, :, 1])
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    micro = rng.integers(0x01, 0x7F, (rows, K // 16)).astype(np.uint8)      # 0x7F (NaN) excluded
    micro[:, ::7] = 0x7E                                                     # 448, the top
    return packed, micro


@pytest.mark.parametrize("M", [16, 128])
def test_nvfp4_gemm_fp16_matrix_core_sums(M):
    """NVFP4 runs on the fp16 matrix cores with each code times its E4M3
    microscale expanded exactly to fp16.  Crafted operands put a product of
    2688 * 2688 next to products of 2^-20 inside one instruction, with
    cancelling pairs: the result must stay within 1e-5 sum_k |x w| (ten times
    inside the contract), which a truncating in-instruction sum like the FP8
    instructions' would break.  M = 16 runs the skinny kernel, M = 128 the
    tiled one."""
    rng = np.random.default_rng(5151 + M)
    N, K = 256, 2048
    a, sa = _crafted_nv(M, K, rng)
    b, sb = _crafted_nv(N, K, rng)
    one = np.ones(1, np.float32)
    label = f"nvfp4 crafted blocks M={M}"
    say(label)
    out = _run(fb.FP4_NV, (a, sa, one, b, sb, one), fb.DT_F32)
    ref, absb = fp4.gemm_ref(fb.FP4_NV, a, sa, b, sb, one[0], one[0])
    gemm_check(out, fb.DT_F32, ref, absb, label, rel=1e-5)
