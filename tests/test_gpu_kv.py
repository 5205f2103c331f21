"""GPU parity: the FP8 KV cache (quantize on append, dequantize on read)
against the oracle, bit for bit: codes in every slot of the pool (untouched
slots included), and the read values in fp32 and bf16.

Cases: both formats, the three scale kinds, fp32 and bf16 inputs, strided
input rows (a slice of a fused QKV output), paged slots in random block order
with padding tokens (slot -1) and slots past the pool, a head size that is not
a power of two (576, as in latent-attention caches), a single token, and the
full-size workload on sampled rows."""

import numpy as np
import pytest
import torch

import block_scaled_precision_x128_amd as fb
import workloads
from oracle import quant
from gpu_helpers import assert_codes_equal, dev, host, say

pytestmark = pytest.mark.gpu

KINDS = [fb.KV_SCALE_TENSOR, fb.KV_SCALE_HEAD, fb.KV_SCALE_CHANNEL]


def _scales(rng, kind, heads, head_dim):
    n = {fb.KV_SCALE_TENSOR: 1, fb.KV_SCALE_HEAD: heads, fb.KV_SCALE_CHANNEL: heads * head_dim}[kind]
    return (np.exp(rng.uniform(-5, 1, n)) / 56).astype(np.float32)


def _bf16_of(y32: np.ndarray) -> np.ndarray:
    return quant.to_bf16_bits(y32)


def _check_gather(cache_d, slots_np, scales_np, fmt, kind, label, want_cache):
    slots_d = dev(slots_np)
    sc_d = dev(scales_np)
    want = quant.kv_gather(want_cache, slots_np, kind, scales_np, fmt)
    y32 = fb.fp8_kv_gather(cache_d, slots_d, sc_d, fmt, kind, fb.DT_F32)
    y16 = fb.fp8_kv_gather(cache_d, slots_d, sc_d, fmt, kind, fb.DT_BF16)
    torch.cuda.synchronize()
    # NaN codes read as NaN; their sign and payload carry no value and are not compared
    g32, w32 = host(y32), want
    nan_g, nan_w = np.isnan(g32), np.isnan(w32)
    assert np.array_equal(nan_g, nan_w), label + " NaN positions (fp32)"
    assert_codes_equal(np.where(nan_g, 0, g32.view(np.uint32)), np.where(nan_w, 0, w32.view(np.uint32)),
                       label + " read fp32")
    g16, w16 = host(y16), _bf16_of(want)
    nan_g, nan_w = (g16 & 0x7FFF) > 0x7F80, (w16 & 0x7FFF) > 0x7F80
    assert np.array_equal(nan_g, nan_w), label + " NaN positions (bf16)"
    assert_codes_equal(np.where(nan_g, 0, g16), np.where(nan_w, 0, w16), label + " read bf16")


@pytest.mark.parametrize("fmt", [fb.E4M3, fb.E5M2])
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dt", [fb.DT_F32, fb.DT_BF16])
def test_kv_append_and_read(fmt, kind, dt):
    rng = np.random.default_rng(300 + 6 * fmt + 2 * kind + dt)
    heads, head_dim, tokens, pool = 4, 80, 157, 240      # 20 chunks a row: rows straddle workgroups
    scales = _scales(rng, kind, heads, head_dim)
    x = (rng.standard_normal((tokens, heads, head_dim)) * np.exp(rng.uniform(-4, 4, (1, heads, head_dim))))
    x = x.astype(np.float32)
    x[3, 1, :5] = [1e30, -1e30, 0.0, -0.0, 3e-30]       # saturation, signed zeros, underflow
    store = workloads.f32_to_bf16_bits(x) if dt == fb.DT_BF16 else x
    x32 = workloads.storage_to_f32(store, dt)
    slots = rng.permutation(pool)[:tokens].astype(np.int64)
    slots[[5, 77]] = -1                                   # padding tokens
    slots[100] = pool + 3                                 # past the pool
    base = rng.integers(0, 256, (pool, heads, head_dim), dtype=np.uint8)
    label = f"kv fmt={fmt} kind={kind} dt={dt} tokens={tokens} pool={pool}"
    say(label)
    cache_d = dev(base)
    fb.fp8_kv_append(dev(store), dev(slots), cache_d, dev(scales), fmt, kind)
    torch.cuda.synchronize()
    want = quant.kv_append(base, x32, slots, kind, scales, fmt)
    assert_codes_equal(host(cache_d), want, label + " cache")
    read = np.concatenate([slots, np.array([-7, pool, 0], np.int64)])
    _check_gather(cache_d, read, scales, fmt, kind, label, want)


@pytest.mark.parametrize("kind", KINDS)
def test_kv_strided_rows_and_wide_heads(kind):
    """x is the K slice of a fused [tokens, q | k | v] projection output;
    heads of 576 (not a power of two)."""
    rng = np.random.default_rng(41 + kind)
    heads, head_dim, tokens, pool = 2, 576, 33, 64
    L = heads * head_dim
    fused = (rng.standard_normal((tokens, 3 * L)) * 3).astype(np.float32)
    fused_b = workloads.f32_to_bf16_bits(fused)
    fused_d = dev(fused_b)
    xk = fused_d[:, L:2 * L].view(tokens, heads, head_dim)
    x32 = workloads.bf16_bits_to_f32(fused_b[:, L:2 * L]).reshape(tokens, heads, head_dim)
    scales = _scales(rng, kind, heads, head_dim)
    slots = rng.permutation(pool)[:tokens].astype(np.int64)
    label = f"kv strided kind={kind} head_dim={head_dim}"
    say(label)
    cache_d = torch.zeros((pool, heads, head_dim), dtype=torch.uint8, device="cuda")
    fb.fp8_kv_append(xk, dev(slots), cache_d, dev(scales), fb.E4M3, kind)
    torch.cuda.synchronize()
    want = quant.kv_append(np.zeros((pool, heads, head_dim), np.uint8), x32, slots, kind, scales, fb.E4M3)
    assert_codes_equal(host(cache_d), want, label + " cache")
    _check_gather(cache_d, slots[::-1].copy(), scales, fb.E4M3, kind, label, want)


def test_kv_decode_step_appends_one_token_per_sequence():
    """A decode step: one new token for each of 32 sequences into a cache that
    already holds their prefix; everything else is left as it was."""
    wl = workloads.KV_CONFIGS["kv_llama8b_b32_ctx8k"]
    rng = np.random.default_rng(9)
    batch, ctx = 32, 48
    pool = workloads.kv_pool_slots(wl, batch, ctx)
    slots_all = workloads.kv_slots(wl, batch, ctx).reshape(batch, ctx)
    scales = workloads.kv_scales(wl)
    prefix = workloads.draw_kv(wl, batch * (ctx - 1), rng)
    step = workloads.draw_kv(wl, batch, rng)
    pre_slots = slots_all[:, :-1].reshape(-1)
    new_slots = slots_all[:, -1].copy()
    say(f"kv decode step batch={batch} ctx={ctx} pool={pool}")
    cache_d = torch.zeros((pool, wl.heads, wl.head_dim), dtype=torch.uint8, device="cuda")
    pb = workloads.f32_to_bf16_bits(prefix)
    sb = workloads.f32_to_bf16_bits(step)
    fb.fp8_kv_append(dev(pb), dev(pre_slots), cache_d, dev(scales), wl.fmt, wl.scale_kind)
    fb.fp8_kv_append(dev(sb), dev(new_slots), cache_d, dev(scales), wl.fmt, wl.scale_kind)
    torch.cuda.synchronize()
    want = np.zeros((pool, wl.heads, wl.head_dim), np.uint8)
    want = quant.kv_append(want, workloads.bf16_bits_to_f32(pb), pre_slots, wl.scale_kind, scales, wl.fmt)
    want = quant.kv_append(want, workloads.bf16_bits_to_f32(sb), new_slots, wl.scale_kind, scales, wl.fmt)
    assert_codes_equal(host(cache_d), want, "decode step cache")
    _check_gather(cache_d, slots_all.reshape(-1), scales, wl.fmt, wl.scale_kind, "decode step", want)


def test_kv_single_token_and_empty():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 1, 16)).astype(np.float32)
    sc = np.array([0.01], np.float32)
    say("kv single token, empty calls")
    cache_d = torch.zeros((3, 1, 16), dtype=torch.uint8, device="cuda")
    fb.fp8_kv_append(dev(x), dev(np.array([2], np.int64)), cache_d, dev(sc), fb.E5M2, fb.KV_SCALE_TENSOR)
    fb.fp8_kv_append(dev(x[:0]), dev(np.zeros(0, np.int64)), cache_d, dev(sc), fb.E5M2, fb.KV_SCALE_TENSOR)
    e = fb.fp8_kv_gather(cache_d, dev(np.zeros(0, np.int64)), dev(sc), fb.E5M2, fb.KV_SCALE_TENSOR)
    torch.cuda.synchronize()
    want = quant.kv_append(np.zeros((3, 1, 16), np.uint8), x, [2], fb.KV_SCALE_TENSOR, sc, fb.E5M2)
    assert_codes_equal(host(cache_d), want, "single token")
    assert e.shape == (0, 1, 16)


def test_kv_full_size_sampled():
    """The benchmark workload (32 sequences x 8192 tokens, 8 heads of 128,
    per-channel E4M3, bf16) in the launch configuration the benchmark times;
    the oracle checks 4096 sampled tokens of the append and of the read."""
    wl = workloads.KV_CONFIGS["kv_llama8b_b32_ctx8k"]
    rng = np.random.default_rng(wl.seed + 7)
    tokens, pool = wl.tokens, workloads.kv_pool_slots(wl)
    slots = workloads.kv_slots(wl)
    scales = workloads.kv_scales(wl)
    say(f"kv full size tokens={tokens} pool={pool}")
    x = torch.randn((tokens, wl.heads, wl.head_dim), device="cuda", dtype=torch.float32)
    x = (x * dev(workloads.kv_sigma(wl))[None]).to(torch.bfloat16)
    cache_d = torch.zeros((pool, wl.heads, wl.head_dim), dtype=torch.uint8, device="cuda")
    fb.fp8_kv_append(x, dev(slots), cache_d, dev(scales), wl.fmt, wl.scale_kind)
    y = fb.fp8_kv_gather(cache_d, dev(slots), dev(scales), wl.fmt, wl.scale_kind, fb.DT_BF16)
    torch.cuda.synchronize()
    pick = np.sort(rng.choice(tokens, 4096, replace=False))
    xs = host(x[torch.from_numpy(pick).cuda()])
    x32 = workloads.bf16_bits_to_f32(xs)
    got_codes = host(cache_d[torch.from_numpy(slots[pick]).cuda()])
    for i in range(0, len(pick), 512):
        want = quant.kv_append(np.zeros((512, wl.heads, wl.head_dim), np.uint8), x32[i:i + 512], np.arange(512),
                               wl.scale_kind, scales, wl.fmt)
        assert_codes_equal(got_codes[i:i + 512], want, f"full size codes, sample block {i}")
        back = quant.kv_gather(want, np.arange(512), wl.scale_kind, scales, wl.fmt)
        assert_codes_equal(host(y[torch.from_numpy(pick[i:i + 512]).cuda()]), _bf16_of(back),
                           f"full size read, sample block {i}")
    # the slots no token maps to are still zero
    free = np.setdiff1d(np.arange(pool), slots)[:2048]
    assert not host(cache_d[torch.from_numpy(free).cuda()]).any()
