"""Seeded synthetic inputs for the FP8 quantize + block-scaled GEMM path.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds input generation only: random draws, outlier injection and
the bf16 storage cast of the inputs.  None of the FP8 method's arithmetic
(amax, scales, FP8 rounding, GEMM) lives here.

The five workloads mirror the shapes and statistics the pages describe:
activations ~N(0,1) with a few outlier channels ten to a hundred times larger
than the rest (page "Illustrated GPU kernels, Part 8", the outlier paragraph
after the qdq listing), weights concentrated near zero with a small spread
(page "FP8 Serving", results section 1), and gradient-like data spanning many
orders of magnitude for the E5M2 operand (page "The FP8 Family", E5M2 row of
the format table).

The FP8 KV-cache workload (KV_CONFIGS) follows page "FP8 Serving" (memory
table row "KV cache (8k, batch 32)" for an 8B model; keys and values carry
channel-structured outliers) with the published Llama 3.1 8B attention shape:
8 KV heads of 128.

Generator recipe (fixed):
  rng = numpy.random.default_rng(seed)            # PCG64
  X   = rng.standard_normal((M, K), float32)
  if outliers: cols = rng.choice(K, n, replace=False); X[:, cols] *= factor
  W   = rng.standard_normal((N, K), float32) * 0.02      (normal weights)
     or sign * 10**rng.uniform(-6, 3, (N, K))            (log-uniform, E5M2)
  bf16 inputs are the fp32 draws rounded to bf16 (round to nearest even).
KV cache:
  channels with outliers: rng.choice(heads * head_dim, n, replace=False) from
  default_rng(seed); sigma = factor there, 1 elsewhere
  values  = rng.standard_normal((tokens, heads, head_dim), float32) * sigma
  slots   = paged: blocks of `block` tokens, a pool of ceil(capacity * tokens /
            block) blocks, sequence blocks = a random permutation of the pool
            (default_rng(seed + 1)); token t of sequence b sits in slot
            perm[b * blocks_per_seq + t // block] * block + t % block
  static scales (given, as a calibration would): sigma / 56 per channel, the
            channel sigma's maximum / 56 per head and per tensor (8 sigma at
            the top of the E4M3 range, 448 = 8 * 56)
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Enum values shared with include/fp8blk.h (plain integers, no arithmetic).
E4M3, E5M2 = 0, 1
GRAN_TENSOR, GRAN_ROW, GRAN_TILE_1x128, GRAN_BLOCK_128x128, GRAN_MX32 = 0, 1, 2, 3, 4
DT_F32, DT_BF16 = 0, 1
KV_SCALE_TENSOR, KV_SCALE_HEAD, KV_SCALE_CHANNEL = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    M: int
    N: int
    K: int
    in_dtype: int          # DT_F32 or DT_BF16 for both X and W
    x_fmt: int
    w_fmt: int
    x_gran: int
    w_gran: int
    out_dtype: int
    x_outlier_frac: float  # fraction of K-columns that are outliers (0 = none)
    x_outlier_factor: float
    w_kind: str            # "normal" (sigma 0.02) or "loguniform" (|w| = 10^U(-6,3))
    x_outlier_count: Optional[int] = None  # exact count when the page fixes it
    fp4_kind: Optional[int] = None         # FP4 workloads: FP4_MX or FP4_NV (formats and granularities unused)

    def n_outliers(self, K: Optional[int] = None) -> int:
        K = self.K if K is None else K
        if self.x_outlier_count is not None and K == self.K:
            return self.x_outlier_count
        return int(round(self.x_outlier_frac * K))

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


# The five configurations of the workload table.
CONFIGS = {
    "c1_per_tensor": Workload(
        "c1_per_tensor", 101, 128, 256, 512, DT_F32, E4M3, E4M3,
        GRAN_TENSOR, GRAN_TENSOR, DT_F32, 0.0, 50.0, "normal", x_outlier_count=2),
    "c2_per_token_channel": Workload(
        "c2_per_token_channel", 102, 2048, 4096, 4096, DT_BF16, E4M3, E4M3,
        GRAN_ROW, GRAN_ROW, DT_BF16, 0.01, 30.0, "normal"),
    "c3_deepseek_block": Workload(
        "c3_deepseek_block", 103, 4096, 7168, 7168, DT_BF16, E4M3, E4M3,
        GRAN_TILE_1x128, GRAN_BLOCK_128x128, DT_BF16, 0.005, 100.0, "normal"),
    "c4_decode_skinny": Workload(
        "c4_decode_skinny", 104, 16, 18432, 7168, DT_BF16, E4M3, E4M3,
        GRAN_TILE_1x128, GRAN_BLOCK_128x128, DT_BF16, 0.0, 1.0, "normal"),
    "c5_mxfp8_mix": Workload(
        "c5_mxfp8_mix", 105, 8192, 8192, 8192, DT_F32, E4M3, E5M2,
        GRAN_MX32, GRAN_MX32, DT_F32, 0.0, 1.0, "loguniform"),
}

CONFIG_ORDER = ["c1_per_tensor", "c2_per_token_channel", "c3_deepseek_block",
                "c4_decode_skinny", "c5_mxfp8_mix"]

# FP4 (E2M1) microscaling at the DeepSeek block-scaled shape and inputs
# ("Illustrated GPU kernels, Part 8": MXFP4 blocks of 32, NVFP4 blocks of 16
# with an E4M3 microscale and a tensor scale).
FP4_MX, FP4_NV = 0, 1
FP4_CONFIGS = {
    "fp4_mx_4096x7168x7168": Workload(
        "fp4_mx_4096x7168x7168", 103, 4096, 7168, 7168, DT_BF16, E4M3, E4M3,
        GRAN_MX32, GRAN_MX32, DT_BF16, 0.005, 100.0, "normal", fp4_kind=FP4_MX),
    "fp4_nv_4096x7168x7168": Workload(
        "fp4_nv_4096x7168x7168", 103, 4096, 7168, 7168, DT_BF16, E4M3, E4M3,
        GRAN_MX32, GRAN_MX32, DT_BF16, 0.005, 100.0, "normal", fp4_kind=FP4_NV),
    # the decode shape and inputs of c4_decode_skinny with MXFP4 / NVFP4 operands
    "fp4_mx_decode_16x18432x7168": Workload(
        "fp4_mx_decode_16x18432x7168", 104, 16, 18432, 7168, DT_BF16, E4M3, E4M3,
        GRAN_MX32, GRAN_MX32, DT_BF16, 0.0, 1.0, "normal", fp4_kind=FP4_MX),
    "fp4_nv_decode_16x18432x7168": Workload(
        "fp4_nv_decode_16x18432x7168", 104, 16, 18432, 7168, DT_BF16, E4M3, E4M3,
        GRAN_MX32, GRAN_MX32, DT_BF16, 0.0, 1.0, "normal", fp4_kind=FP4_NV),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns.

    Storage cast of the synthetic inputs (finite values only)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def draw_x(wl: Workload, rows: Optional[int] = None, cols: Optional[int] = None,
           rng: Optional[np.random.Generator] = None) -> np.ndarray:
    """Activation operand as fp32 values, before the storage cast."""
    rows = wl.M if rows is None else rows
    cols = wl.K if cols is None else cols
    rng = np.random.default_rng(wl.seed) if rng is None else rng
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    n = wl.n_outliers(cols)
    if n > 0:
        idx = rng.choice(cols, n, replace=False)
        x[:, idx] *= np.float32(wl.x_outlier_factor)
    return x


def draw_w(wl: Workload, rows: Optional[int] = None, cols: Optional[int] = None,
           rng: Optional[np.random.Generator] = None) -> np.ndarray:
    """Weight operand as fp32 values, before the storage cast."""
    rows = wl.N if rows is None else rows
    cols = wl.K if cols is None else cols
    rng = np.random.default_rng(wl.seed + 1000) if rng is None else rng
    if wl.w_kind == "normal":
        return rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(0.02)
    mag = np.power(10.0, rng.uniform(-6.0, 3.0, size=(rows, cols)))
    sign = np.where(rng.integers(0, 2, size=(rows, cols)) == 1, 1.0, -1.0)
    return (sign * mag).astype(np.float32)


def make_inputs(wl: Workload, M: Optional[int] = None, N: Optional[int] = None,
                K: Optional[int] = None, seed_offset: int = 0):
    """Return (x_store, w_store) in the workload's storage dtype.

    fp32 workloads give float32 arrays; bf16 workloads give uint16 bf16 bit
    patterns.  M/N/K override the shape (for reduced-size parity cases); one
    generator stream is used so that X is drawn before W.
    """
    M = wl.M if M is None else M
    N = wl.N if N is None else N
    K = wl.K if K is None else K
    rng = np.random.default_rng(wl.seed + seed_offset)
    x = draw_x(wl, M, K, rng)
    w = draw_w(wl, N, K, rng)
    if wl.in_dtype == DT_BF16:
        return f32_to_bf16_bits(x), f32_to_bf16_bits(w)
    return x, w


def storage_to_f32(a: np.ndarray, dtype: int) -> np.ndarray:
    """Exact fp32 values of a stored operand."""
    if dtype == DT_BF16:
        return bf16_bits_to_f32(a)
    return np.asarray(a, dtype=np.float32)


# ---- FP8 KV cache --------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class KvWorkload:
    name: str
    seed: int
    batch: int
    context: int           # tokens per sequence
    heads: int             # KV heads
    head_dim: int
    block: int             # paged-cache block, tokens
    capacity: float        # pool slots / tokens held
    fmt: int
    scale_kind: int
    in_dtype: int
    out_dtype: int
    outlier_frac: float    # fraction of channels with outliers
    outlier_factor: float  # their sigma

    @property
    def tokens(self) -> int:
        return self.batch * self.context

    @property
    def row(self) -> int:
        return self.heads * self.head_dim

    @property
    def blocks_per_seq(self) -> int:
        return -(-self.context // self.block)


KV_CONFIGS = {
    "kv_llama8b_b32_ctx8k": KvWorkload(
        "kv_llama8b_b32_ctx8k", 201, 32, 8192, 8, 128, 16, 1.25, E4M3, KV_SCALE_CHANNEL, DT_BF16, DT_BF16,
        1.0 / 64, 20.0),
}


def kv_sigma(wl: KvWorkload) -> np.ndarray:
    """Per-channel standard deviation [heads, head_dim]."""
    rng = np.random.default_rng(wl.seed)
    sig = np.ones(wl.row, np.float32)
    n = int(round(wl.outlier_frac * wl.row))
    if n > 0:
        sig[rng.choice(wl.row, n, replace=False)] = np.float32(wl.outlier_factor)
    return sig.reshape(wl.heads, wl.head_dim)


def draw_kv(wl: KvWorkload, tokens: int, rng: np.random.Generator) -> np.ndarray:
    """Key or value states [tokens, heads, head_dim] as fp32 values."""
    return rng.standard_normal((tokens, wl.heads, wl.head_dim), dtype=np.float32) * kv_sigma(wl)[None]


def kv_slots(wl: KvWorkload, batch: Optional[int] = None, context: Optional[int] = None) -> np.ndarray:
    """Slot of every token, sequence-major ([batch * context] int64), for a
    paged pool whose blocks are handed out in a random order."""
    batch = wl.batch if batch is None else batch
    context = wl.context if context is None else context
    bps = -(-context // wl.block)
    pool = max(int(np.ceil(wl.capacity * batch * bps)), batch * bps)
    perm = np.random.default_rng(wl.seed + 1).permutation(pool)[: batch * bps].reshape(batch, bps)
    t = np.arange(context)
    slots = perm[:, t // wl.block] * wl.block + (t % wl.block)[None, :]
    return slots.reshape(-1).astype(np.int64)


def kv_pool_slots(wl: KvWorkload, batch: Optional[int] = None, context: Optional[int] = None) -> int:
    batch = wl.batch if batch is None else batch
    context = wl.context if context is None else context
    bps = -(-context // wl.block)
    return max(int(np.ceil(wl.capacity * batch * bps)), batch * bps) * wl.block


def kv_scales(wl: KvWorkload, scale_kind: Optional[int] = None) -> np.ndarray:
    """Static scales of the given kind (float32 [1], [heads] or [heads * head_dim])."""
    kind = wl.scale_kind if scale_kind is None else scale_kind
    sig = kv_sigma(wl)
    if kind == KV_SCALE_CHANNEL:
        return (sig / np.float32(56.0)).reshape(-1).astype(np.float32)
    if kind == KV_SCALE_HEAD:
        return (sig.max(axis=1) / np.float32(56.0)).astype(np.float32)
    return np.array([sig.max() / np.float32(56.0)], np.float32)
