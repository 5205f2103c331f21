#!/usr/bin/env python3
"""Throughput of the FP8 quantize + block-scaled GEMM path on one MI355X.

One step = the whole hot path over one batch of synthetic input that is
already resident in HBM:
    quantize X (bf16 -> E4M3, fp32 scale per 1x128 tile)
    quantize W (bf16 -> E4M3, fp32 scale per 128x128 block)
    GEMM  out = sum_kb sX[m,kb] sW[n/128,kb] (X_kb @ W_kb^T), bf16 out
    dequantize X (the activation round trip, codes -> bf16)
on the DeepSeek-V3-style block-scaled workload M=4096, N=7168, K=7168.
`value` is 2*M*N*K / (time per step) in TFLOP/s.

Timing: after --warmup eager steps, 5 batches of exactly --steps steps, each
enqueued behind a spin kernel (so the launches run back to back, with no
host gaps) and an untimed pre-roll of >= 25 ms of the same steps (so they run
at the engine clock a sustained load holds: right after an idle spin the
clock is low for the first milliseconds), each bracketed by HIP events on the
launch stream and device synchronizes; ms_per_step is the median batch.
Each kernel is timed on its own the same way: the
dominant kernel (the GEMM) against the fp8 matrix-core peak (the metric's
denominator; the exact default multiplies on the bf16 matrix cores, half that
rate, and its fraction of the bf16 peak is reported beside it) or, for the
decode workload, against the HBM peak; quantize and dequantize in algorithmic
GB/s against the HBM peak.  The default run also times the kernels of the other
four workloads (c1, c2, c4, c5; no CPU leg), the machine's own ceilings
(back-to-back MFMAs, a streaming read, a device copy: include/fp8blk_probe.h)
and reads the GPU clock levels from sysfs when it can.

Input sets are rotated so that every kernel moving 8 MB or more per launch
cycles at least 640 MB of its own data (2.5x the 256 MB last-level cache):
no timed launch reads what an earlier launch left in that cache.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--accum fp32|native] [--no-cpu-baseline] [--no-other-configs]
                    [--no-ceilings] [--copy-probe]

For the decode workload (c4_decode_skinny) W is quantized once per input set
in setup, as a model's weights are, and a step is quantize X + GEMM + dequantize X.

The FP4 workloads (--workload fp4_mx_4096x7168x7168 / fp4_nv_4096x7168x7168:
the DeepSeek shape and inputs with E2M1 operands, MXFP4 or NVFP4 scales) run
quantize X + quantize W + GEMM + dequantize X the same way.  The FP4 decode
workloads (--workload fp4_mx_decode_16x18432x7168 / fp4_nv_decode_16x18432x7168:
c4's shape and inputs) quantize W in setup, like c4, and report the GEMM
against HBM.

The FP8 KV-cache workload (--workload kv_llama8b_b32_ctx8k: 32 sequences of
8192 tokens, 8 KV heads of 128, bf16 states, E4M3 codes with per-channel
scales, a paged pool in random block order) has a step of its own: append
the keys and the values of every token (quantize on append), then read both
back to bf16 (dequantize on read); `value` is tokens per second and the
roofline is the HBM bound of the longer of the two kernels.

Profiling helpers (no GPU needed; they read rocprofv3 output):
    python bench.py --summarize-trace DIR       kernel-trace --stats summary
    python bench.py --summarize-traffic ...     HBM bytes of the GEMM from two
                                                --pmc runs, calibrated by a copy
`roofline.traffic` is filled from profiles/traffic_<workload>_<accum>.txt when
that file was taken from the GEMM sources as they are now (a SHA-256 of them
is stored in it), and is null otherwise.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "block-scaled FP8 GEMM TFLOP/s (% fp8 MFMA peak); quantize GB/s (% HBM)"
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 matrix-core peak
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 matrix-core peak
PEAK_FP4_TFLOPS = 10100.0    # MI355X dense fp4 matrix-core peak
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E peak
COPY_PROBE_BYTES = 256 << 20  # size of the plain copy that calibrates the byte counters


def scale_bytes(gran: int, rows: int, cols: int) -> int:
    return {workloads.GRAN_TENSOR: 4, workloads.GRAN_ROW: 4 * rows,
            workloads.GRAN_TILE_1x128: 4 * rows * (cols // 128),
            workloads.GRAN_BLOCK_128x128: 4 * (rows // 128) * (cols // 128),
            workloads.GRAN_MX32: rows * (cols // 32)}[gran]


def quant_bytes(wl, operand: str) -> int:
    """Algorithmic bytes of one quantize: input read once, codes and scales written."""
    rows, cols = (wl.M, wl.K) if operand == "x" else (wl.N, wl.K)
    gran = wl.x_gran if operand == "x" else wl.w_gran
    in_b = 2 if wl.in_dtype == workloads.DT_BF16 else 4
    return rows * cols * (in_b + 1) + scale_bytes(gran, rows, cols)


def dequant_bytes(wl) -> int:
    """Algorithmic bytes of dequantizing X: codes and scales read, values written in the input dtype."""
    out_b = 2 if wl.in_dtype == workloads.DT_BF16 else 4
    return wl.M * wl.K * (1 + out_b) + scale_bytes(wl.x_gran, wl.M, wl.K)


def gemm_bytes(wl) -> int:
    """Algorithmic bytes of one GEMM: both code operands and scales read once, output written once."""
    out_b = 2 if wl.out_dtype == workloads.DT_BF16 else 4
    return (wl.M * wl.K + wl.N * wl.K + scale_bytes(wl.x_gran, wl.M, wl.K)
            + scale_bytes(wl.w_gran, wl.N, wl.K) + wl.M * wl.N * out_b)


# Each kernel timed on rotated inputs cycles at least this many bytes of its
# own data, 2.5x the 256 MB last-level cache, so that no timed launch reads
# what an earlier one left there.
ROTATION_BYTES = 640e6


def rotation_sets(wl) -> int:
    """Input sets to rotate over: enough that every kernel moving 8 MB or
    more per launch (smaller ones are bound by launch latency) cycles
    ROTATION_BYTES of its own data, at most 32."""
    sizes = [quant_bytes(wl, "x"), gemm_bytes(wl), dequant_bytes(wl)]
    if wl.M > 64:
        sizes.append(quant_bytes(wl, "w"))
    big = [b for b in sizes if b >= 8e6]
    return int(min(32, max(2, np.ceil(ROTATION_BYTES / min(big))))) if big else 2


def cpu_baseline(wl, sample_rows: int):
    """The oracle on the host over the same step: quantize a sample of X rows
    and all of W, the fp64 GEMM (Ref and the |x||w| bound) of those rows, and
    the dequantize of the X codes; TFLOP/s of the sample's 2*rows*N*K."""
    from oracle import gemm as ogemm
    from oracle import quant as oquant
    threads = blas_threads()
    xs, ws = workloads.make_inputs(wl, M=sample_rows)
    x = workloads.storage_to_f32(xs, wl.in_dtype)
    w = workloads.storage_to_f32(ws, wl.in_dtype)
    t0 = time.perf_counter()
    xq, sx = oquant.quantize(x, wl.x_gran, wl.x_fmt)
    wq, sw = oquant.quantize(w, wl.w_gran, wl.w_fmt)
    ref, absb = ogemm.gemm_ref(xq, sx, wl.x_gran, wl.x_fmt, wq, sw, wl.w_gran, wl.w_fmt)
    oquant.dequantize(xq, sx, wl.x_gran, wl.x_fmt)
    dt = time.perf_counter() - t0
    flops = 2.0 * sample_rows * wl.N * wl.K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": host_cores(), "kind": "oracle",
            "blas_threads": int(threads), "quantize_threads": 1,
            "sample": f"{sample_rows} of {wl.M} rows of X with all of W: oracle quantize of both operands, "
                      f"fp64 GEMM and bound, dequantize of X; {dt:.2f} s on {host_cores()} host cores "
                      f"(numpy BLAS threads={threads} for the GEMM, the quantize and dequantize on 1 thread)"}


GEMM_SOURCES = ("gemm.hip", "gemm_skinny.hip", "gemm_common.h", "device_common.h", "kernels.h")
KV_SOURCES = ("kv_cache.hip", "kv_cache.h", "given_scale.h", "gemm_common.h", "device_common.h")


def gemm_source_hash(sources=GEMM_SOURCES) -> str:
    """SHA-256 over the kernel sources (counter summaries are valid only for these)."""
    import hashlib
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "block_scaled_precision_x128_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_path(workload: str, accum: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}_{accum}.txt")


def read_traffic(workload: str, accum: str, sources=GEMM_SOURCES):
    """HBM bytes per launch from a stored counter summary, or None when there
    is none or it was taken from other kernel sources."""
    path = traffic_path(workload, accum)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != gemm_source_hash(sources) or "traffic_bytes_per_launch" not in kv:
        return None
    return int(float(kv["traffic_bytes_per_launch"]))


def _sqlite_db(d: str) -> str:
    import glob
    dbs = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))
    if not dbs:
        raise SystemExit(f"no rocprofv3 database under {d}")
    return dbs[0]


def summarize_trace(d: str) -> str:
    """Per-kernel call count and mean/total duration from a rocprofv3
    --kernel-trace --stats database, one line per kernel and grid size (a
    kernel launched on problems of different sizes gets a line for each)."""
    import sqlite3
    con = sqlite3.connect(_sqlite_db(d))
    rows = list(con.execute("select name, grid_x, count(*), sum(duration), avg(duration) from kernels "
                            "group by name, grid_x order by sum(duration) desc"))
    total = sum(r[3] for r in rows) or 1
    out = [f"{'calls':>6} {'mean_us':>10} {'total_us':>11} {'pct':>6} {'grid':>9}  kernel"]
    for name, grid, calls, tot, avg in rows:
        # durations are in nanoseconds
        out.append(f"{calls:6d} {avg / 1e3:10.2f} {tot / 1e3:11.1f} {100 * tot / total:6.2f} {grid:9d}  {name}")
    return "\n".join(out)


def _pmc_rows(path: str, counter: str, min_grid: int = 0):
    import csv
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter and int(float(r.get("Grid_Size") or 0)) >= min_grid:
                rows.append((r.get("Kernel_Name", ""), float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no {counter} rows in {path}")
    return rows


# The GEMM kernels of a plain launch: f32 or bf16 output (the fourth template
# argument, 0 or 1).  The quantized-output variant (2, 3) is a different launch.
GEMM_KERNEL_RE = r"k_gemm_\w+<\d+, \d+, \d+, [01],"


def summarize_traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, kernel_re, copy_bytes,
                      sources=GEMM_SOURCES, min_grid: int = 0):
    """HBM bytes per launch of the kernels whose name matches kernel_re:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) averaged over the dispatches
    of each distinct kernel, summed over those kernels (one launch runs each of
    them once: the column split's two tile shapes), each counter scaled by
    (known bytes / counter reading) of a plain device copy."""
    import re
    pat = re.compile(kernel_re)

    def per_kernel(path, counter):
        by = {}
        for n, v in _pmc_rows(path, counter, min_grid):
            if pat.search(n):
                by.setdefault(n, []).append(v)
        if not by:
            raise SystemExit(f"no {counter} dispatch of the selected kernels in {path}")
        return {n: float(np.mean(v)) for n, v in by.items()}, sum(len(v) for v in by.values())

    fetch, nf = per_kernel(fetch_csv, "FETCH_SIZE")
    write, nw = per_kernel(write_csv, "WRITE_SIZE")
    if set(fetch) != set(write):
        raise SystemExit("FETCH_SIZE and WRITE_SIZE runs saw different kernels")
    fk, wk = sum(fetch.values()), sum(write.values())
    # the copy probe's copy is its largest dispatch
    cf = max(v for _, v in _pmc_rows(copy_fetch_csv, "FETCH_SIZE"))
    cw = max(v for _, v in _pmc_rows(copy_write_csv, "WRITE_SIZE"))
    kib = copy_bytes / 1024.0
    ff, fw = kib / cf, kib / cw
    traffic = (fk * ff + wk * fw) * 1024.0
    lines = [f"kernel_match: {kernel_re}"] + ([f"min_grid: {min_grid}"] if min_grid else [])
    for n in sorted(fetch):
        lines.append(f"  kernel {n}: fetch_kib {fetch[n]:.1f}, write_kib {write[n]:.1f} (mean per dispatch)")
    lines += [
        f"fetch_kib_per_launch: {fk:.1f}   ({len(fetch)} kernel(s), {nf} dispatches)",
        f"write_kib_per_launch: {wk:.1f}   ({len(write)} kernel(s), {nw} dispatches)",
        f"copy_bytes: {copy_bytes}",
        f"copy_fetch_kib: {cf:.1f}",
        f"copy_write_kib: {cw:.1f}",
        f"fetch_factor: {ff:.4f}",
        f"write_factor: {fw:.4f}",
        f"traffic_bytes_per_launch: {traffic:.0f}",
        f"source_sha256: {gemm_source_hash(sources)}",
    ]
    return "\n".join(lines)


def summarize_counters(csv_paths, kernel_re, sources=GEMM_SOURCES) -> str:
    """Per-kernel means over dispatches of every counter found in the given
    rocprofv3 --pmc CSV files (one pass each), and the figures derived from
    them: instructions per wave and per MFMA instruction."""
    import csv
    import re
    pat = re.compile(kernel_re)
    vals = {}   # kernel -> counter -> [values]
    grids = {}
    for path in csv_paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                n = r.get("Kernel_Name", "")
                if not pat.search(n):
                    continue
                vals.setdefault(n, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                grids[n] = int(float(r.get("Grid_Size") or 0))
    if not vals:
        raise SystemExit("no dispatch of the selected kernels in " + ", ".join(csv_paths))
    lines = [f"kernel_match: {kernel_re}"]
    for n in sorted(vals):
        c = {k: float(np.mean(v)) for k, v in vals[n].items()}
        waves = grids[n] / 64.0
        lines.append(f"kernel {n}  (grid {grids[n]} threads = {waves:.0f} waves)")
        for k in sorted(c):
            lines.append(f"  {k}: {c[k]:.6g}   ({len(vals[n][k])} dispatches)")
        mf = c.get("SQ_INSTS_MFMA")
        if mf:
            for k in ("SQ_INSTS_VALU", "SQ_INSTS_VALU_CVT", "SQ_INSTS_VALU_FMA_F32", "SQ_INSTS_VALU_MUL_F32",
                      "SQ_INSTS_LDS", "SQ_INSTS_VMEM", "SQ_INSTS_SALU"):
                if k in c:
                    lines.append(f"  per MFMA instruction {k}: {c[k] / mf:.3f}")
            if "SQ_INSTS_VALU" in c:
                lines.append(f"  per MFMA instruction non-MFMA VALU: {(c['SQ_INSTS_VALU'] - mf) / mf:.3f}"
                             "   (SQ_INSTS_VALU counts the MFMAs too)")
            lines.append(f"  MFMA instructions per wave: {mf / waves:.1f}")
    lines.append(f"source_sha256: {gemm_source_hash(sources)}")
    return "\n".join(lines)


# ---- timing -------------------------------------------------------------------

class Timer:
    """Times a unit of GPU work enqueued by a Python callable.

    `enqueue(i, stream)` enqueues iteration i (which rotates over the input
    sets) on `stream`.  Each batch is enqueued eagerly behind a spin kernel
    that keeps the GPU busy while the host queues the launches, so the timed
    launches run back to back with no host gaps; between the spin and the
    timed launches sits an untimed pre-roll of the same work lasting at least
    `preroll_ms` (at most 400 iterations), so the timed launches start at the
    engine clock a sustained load runs at: after a spin or an idle host the
    c3 GEMM starts about 20% slower and needs 30-40 ms of back-to-back work to
    reach its steady rate (per-launch events).  HIP events on the launch stream bracket exactly `reps`
    iterations; the device is synchronized before and after each batch.
    """

    def __init__(self, torch, preroll_ms: float = 60.0):
        self.torch = torch
        self.preroll_ms = preroll_ms
        st = torch.cuda.current_stream()
        torch.cuda._sleep(1_000_000)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        torch.cuda._sleep(4_000_000)
        e1.record(st)
        torch.cuda.synchronize()
        self.cycles_per_ms = 4_000_000 / max(e0.elapsed_time(e1), 1e-3)

    def batches(self, enqueue, reps: int, nbatch: int = 5):
        torch = self.torch
        st = torch.cuda.current_stream()
        # estimate the GPU time and the host enqueue time of one iteration
        torch.cuda.synchronize()
        n0 = max(2, min(reps, 8))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        h0 = time.perf_counter()
        e0.record(st)
        for i in range(n0):
            enqueue(i, st)
        e1.record(st)
        host_ms = (time.perf_counter() - h0) * 1e3 / n0
        torch.cuda.synchronize()
        gpu_ms = max(e0.elapsed_time(e1) / n0, 1e-3)
        # at most 400 pre-roll iterations: queued work past the stream's hardware
        # queue blocks the host, and work shorter than its own launch cost then
        # runs at the host's enqueue rate (a 4.8 us KV decode append measured
        # 23.5 us with 3000 iterations; c1's two-launch per-tensor quantize,
        # 8 us of GPU time, measured 19 us with 1000)
        pre = int(min(400, max(2, np.ceil(self.preroll_ms / gpu_ms))))
        spin_ms = min(3000.0, 1.5 * host_ms * (pre + reps) + 1.0)
        out = []
        for _ in range(nbatch):
            torch.cuda.synchronize()
            torch.cuda._sleep(int(spin_ms * self.cycles_per_ms))
            for i in range(pre):
                enqueue(reps + i, st)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for i in range(reps):
                enqueue(i, st)
            e1.record(st)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / reps)
        return out


def median(xs):
    return float(np.median(np.asarray(xs, dtype=np.float64)))


def host_cores() -> int:
    """Host cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return 1


def gpu_clocks():
    """Engine and memory clock levels the driver reports (sysfs), if readable."""
    import glob
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        for key, name in (("pp_dpm_sclk", "sclk"), ("pp_dpm_mclk", "mclk")):
            try:
                with open(os.path.join(dev, key)) as f:
                    lines = [ln.strip() for ln in f if ln.strip()]
            except OSError:
                continue
            cur = [ln for ln in lines if ln.endswith("*")]
            out.setdefault(os.path.basename(os.path.dirname(dev)), {})[name] = {
                "levels": [ln.split(":", 1)[1].strip().rstrip("*").strip() for ln in lines],
                "current": cur[0].split(":", 1)[1].strip().rstrip("*").strip() if cur else None}
    return out or None


def measure_ceilings(torch, fb, timer, reps: int):
    """The machine's own ceilings beside the published peaks: back-to-back
    MFMAs (bf16 and fp8, 2 waves per SIMD as the tiled GEMM runs, and 1), a
    streaming read and a device copy of 1 GiB (4x the last-level cache)."""
    res = {}
    sink = torch.empty(int(fb.load_library().fp8blk_probe_mfma_sink_floats(2)), dtype=torch.float32, device="cuda")
    for kind, name in ((fb.PROBE_MFMA_BF16, "bf16"), (fb.PROBE_MFMA_FP8, "fp8")):
        for wps in (2, 1):
            iters = 2000
            flops = fb.probe_mfma(kind, wps, iters, sink)
            ms = median(timer.batches(lambda i, st: fb.probe_mfma(kind, wps, iters, sink, stream=st), reps=5))
            res[f"mfma_{name}_{wps}wave_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(3)
    dst = torch.empty_like(src)
    rsink = torch.empty(int(fb.load_library().fp8blk_probe_read_sink_floats()), dtype=torch.float32, device="cuda")
    ms = median(timer.batches(lambda i, st: fb.probe_read(src, rsink, stream=st), reps=max(3, reps // 4)))
    res["read_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    ms = median(timer.batches(lambda i, st: fb.probe_copy(src, dst, stream=st), reps=max(3, reps // 4)))
    res["copy_gbs"] = round(2 * nbytes / (ms * 1e-3) / 1e9, 1)
    res["note"] = ("median of 5 batches timed like the kernels; mfma_*: 8 independent accumulator chains per wave, "
                   "one workgroup per CU; read: 1 GiB streamed once; copy: 1 GiB read + 1 GiB written")
    del src, dst
    return res


class SizedCeilings:
    """The read and copy probes at the byte volume of a given kernel, so that a
    kernel moving tens of megabytes is priced against what a plain stream of
    the same size reaches (launch, ramp-up and drain weigh more there than in
    the 1 GiB figures).  Each iteration takes the next disjoint slice of two
    1 GiB buffers, so the slices cycled over exceed the 256 MB last-level
    cache as the kernels' rotated input sets do.  copy: half the bytes read,
    half written (the quantize and dequantize kernels read 2:1 or 1:2)."""

    def __init__(self, torch, fb, timer, reps: int):
        self.fb, self.timer, self.reps = fb, timer, max(5, reps)
        self.src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(3)
        self.dst = torch.empty_like(self.src)
        self.sink = torch.empty(int(fb.load_library().fp8blk_probe_read_sink_floats()), dtype=torch.float32,
                                device="cuda")
        self.cache = {}

    def gbs(self, kind: str, total_bytes: int) -> float:
        n = (total_bytes // 2 if kind == "copy" else total_bytes) // 4096 * 4096
        n = max(4096, min(n, 1 << 30))
        if (kind, n) not in self.cache:
            slots = max(1, (1 << 30) // n)
            src, dst, sink, fb = self.src, self.dst, self.sink, self.fb
            if kind == "copy":
                f = lambda i, st: fb.probe_copy(src[(i % slots) * n:(i % slots + 1) * n],
                                                dst[(i % slots) * n:(i % slots + 1) * n], stream=st)
            else:
                f = lambda i, st: fb.probe_read(src[(i % slots) * n:(i % slots + 1) * n], sink, stream=st)
            ms = median(self.timer.batches(f, self.reps))
            self.cache[(kind, n)] = (2 if kind == "copy" else 1) * n / (ms * 1e-3) / 1e9
        return self.cache[(kind, n)]

    def annotate(self, kern: dict, wl):
        """Adds <kernel>_ceiling_gbs and <kernel>_frac_ceiling for the
        HBM-bound kernels of a workload's figures."""
        items = [("quantize_x", quant_bytes(wl, "x"), "copy"), ("quantize_w", quant_bytes(wl, "w"), "copy"),
                 ("dequantize_x", dequant_bytes(wl), "copy")]
        if "quantize_x_delayed_gbs" in kern:
            in_b = 2 if wl.in_dtype == workloads.DT_BF16 else 4
            items.append(("quantize_x_delayed", wl.M * wl.K * (in_b + 1) + 8, "copy"))
        for key, nbytes, kind in items:
            g = self.gbs(kind, nbytes)
            kern[f"{key}_ceiling_gbs"] = round(g, 1)
            kern[f"{key}_frac_ceiling"] = round(kern[f"{key}_gbs"] / g, 4)
        if wl.M <= 64:   # decode: the GEMM streams W once
            g = self.gbs("read", gemm_bytes(wl))
            kern["gemm_ceiling_gbs"] = round(g, 1)
            kern["gemm_frac_ceiling"] = round(kern["gemm_algorithmic_gbs"] / g, 4)


# ---- FP8 KV cache ----------------------------------------------------------

def kv_bytes(wl, op: str) -> int:
    """Algorithmic bytes of one append or read of every token: the values
    (bf16/fp32) once, the codes once, 8 bytes of slot per token, the scales."""
    n = wl.tokens * wl.row
    val_b = (2 if (wl.in_dtype if op == "append" else wl.out_dtype) == workloads.DT_BF16 else 4)
    sc = {workloads.KV_SCALE_TENSOR: 1, workloads.KV_SCALE_HEAD: wl.heads,
          workloads.KV_SCALE_CHANNEL: wl.row}[wl.scale_kind]
    return n * (val_b + 1) + 8 * wl.tokens + 4 * sc


def kv_cpu_baseline(wl, sample_tokens: int):
    """The oracle on the host: append and read back a sample of tokens, for
    keys and values; tokens per second."""
    from oracle import quant as oquant
    rng = np.random.default_rng(wl.seed)
    x = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(workloads.draw_kv(wl, sample_tokens, rng)))
    slots = np.arange(sample_tokens, dtype=np.int64)
    scales = workloads.kv_scales(wl)
    cache = np.zeros((sample_tokens, wl.heads, wl.head_dim), np.uint8)
    t0 = time.perf_counter()
    c = oquant.kv_append(cache, x, slots, wl.scale_kind, scales, wl.fmt)
    y = oquant.kv_gather(c, slots, wl.scale_kind, scales, wl.fmt)
    oquant.to_bf16_bits(y)
    dt = 2 * (time.perf_counter() - t0)          # keys and values
    return {"value": sample_tokens / dt, "unit": "tokens/s", "cores": host_cores(), "kind": "oracle",
            "threads_used": 1,
            "sample": f"{sample_tokens} of {wl.tokens} tokens: oracle append (quantize) and read (dequantize "
                      f"to bf16) of one tensor, timed {dt / 2:.2f} s and doubled for keys and values; 1 thread"}


def bench_kv(args, wl) -> int:
    import torch
    import block_scaled_precision_x128_amd as fb

    fb.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    T, H, D = wl.tokens, wl.heads, wl.head_dim
    pool = workloads.kv_pool_slots(wl)
    slots = torch.from_numpy(workloads.kv_slots(wl)).to(dev)
    sig = torch.from_numpy(workloads.kv_sigma(wl)).to(dev)
    scales = {k: torch.from_numpy(workloads.kv_scales(wl, k)).to(dev)
              for k in (fb.KV_SCALE_TENSOR, fb.KV_SCALE_HEAD, fb.KV_SCALE_CHANNEL)}
    sc = scales[wl.scale_kind]
    # States drawn on the GPU (same distribution as the recipe, torch's stream).
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    in_dt = torch.bfloat16 if wl.in_dtype == workloads.DT_BF16 else torch.float32
    out_dt = torch.bfloat16 if wl.out_dtype == workloads.DT_BF16 else torch.float32
    states = [(torch.randn((T, H, D), generator=gen, device=dev) * sig[None]).to(in_dt) for _ in range(2)]
    caches = [torch.zeros((pool, H, D), dtype=torch.uint8, device=dev) for _ in range(2)]
    outs = [torch.empty((T, H, D), dtype=out_dt, device=dev) for _ in range(2)]

    def append(i, kind=None, s=None):
        k = wl.scale_kind if kind is None else kind
        fb.fp8_kv_append(states[i % 2], slots, caches[i % 2], scales[k], wl.fmt, k, stream=s)

    def read(i, kind=None, s=None):
        k = wl.scale_kind if kind is None else kind
        fb.fp8_kv_gather(caches[i % 2], slots, scales[k], wl.fmt, k, wl.out_dtype, out=outs[i % 2], stream=s)

    def step(_, s):
        append(0, s=s)
        append(1, s=s)
        read(0, s=s)
        read(1, s=s)

    for i in range(args.warmup):
        step(i, stream)
    torch.cuda.synchronize()
    timer = Timer(torch, preroll_ms=args.preroll_ms)
    wall0 = time.perf_counter()
    step_batches = timer.batches(step, args.steps)
    wall = time.perf_counter() - wall0
    ms_step = median(step_batches)
    app_ms = median(timer.batches(lambda i, s: append(i, s=s), args.steps))
    rd_ms = median(timer.batches(lambda i, s: read(i, s=s), args.steps))
    per_kind = {}
    for name, k in (("tensor", fb.KV_SCALE_TENSOR), ("head", fb.KV_SCALE_HEAD), ("channel", fb.KV_SCALE_CHANNEL)):
        per_kind[name] = {"append_ms": round(median(timer.batches(lambda i, s: append(i, k, s), args.steps)), 4),
                          "read_ms": round(median(timer.batches(lambda i, s: read(i, k, s), args.steps)), 4)}
    # a decode step: one new token for each sequence
    last = slots.view(wl.batch, wl.context)[:, -1].contiguous()
    new = states[0].view(wl.batch, wl.context, H, D)[:, -1].contiguous()
    dec_ms = median(timer.batches(lambda i, s: fb.fp8_kv_append(new, last, caches[0], sc, wl.fmt, wl.scale_kind,
                                                                 stream=s), max(args.steps, 50)))
    # leave the caches as the step writes them
    step(0, stream)
    torch.cuda.synchronize()

    app_gbs = kv_bytes(wl, "append") / (app_ms * 1e-3) / 1e9
    rd_gbs = kv_bytes(wl, "read") / (rd_ms * 1e-3) / 1e9
    dom = "append" if app_ms >= rd_ms else "read"
    dom_gbs = app_gbs if dom == "append" else rd_gbs
    traffic = read_traffic(wl.name, dom, KV_SOURCES)
    result = {
        "metric": "FP8 KV-cache tokens/s (append + read of keys and values)",
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic (seeded; bf16 states ~N(0,1) with channel outliers x20, drawn on the GPU)",
        "config": {"workload": f"{wl.name}: {wl.batch} sequences x {wl.context} tokens, {H} KV heads x {D}, "
                               f"paged blocks of {wl.block} in random order, pool {pool} slots, E4M3, "
                               f"per-channel scales, bf16 in and out",
                   "step": "append keys + append values + read keys + read values (all tokens)",
                   "cache_bytes_fp8": 2 * pool * wl.row, "cache_bytes_bf16_equivalent": 4 * pool * wl.row},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(dom_gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(dom_gbs / PEAK_HBM_GBS, 4), "traffic": traffic},
        "kernels": {"append_ms": round(app_ms, 4), "append_gbs": round(app_gbs, 1),
                    "append_frac_hbm": round(app_gbs / PEAK_HBM_GBS, 4),
                    "read_ms": round(rd_ms, 4), "read_gbs": round(rd_gbs, 1),
                    "read_frac_hbm": round(rd_gbs / PEAK_HBM_GBS, 4),
                    "by_scale_kind": per_kind,
                    "decode_append_us": round(dec_ms * 1e3, 2)},
        "step_batches_ms": [round(x, 4) for x in step_batches],
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = kv_cpu_baseline(wl, args.kv_cpu_sample_tokens)
    print(json.dumps(result), flush=True)
    return 0


# ---- FP4 (E2M1) microscaling --------------------------------------------------

def fp4_cpu_baseline(wl, x_rows: int, w_rows: int):
    """The oracle on the host: FP4 quantize of a sample of X and W rows, the
    fp64 GEMM of the sample, dequantize of the X sample; TFLOP/s of 2 m n K."""
    from oracle import fp4 as ofp4
    xs, ws = workloads.make_inputs(wl, M=x_rows, N=w_rows)
    x = workloads.storage_to_f32(xs, wl.in_dtype)
    w = workloads.storage_to_f32(ws, wl.in_dtype)
    t0 = time.perf_counter()
    if wl.fp4_kind == workloads.FP4_MX:
        a, sa = ofp4.quantize_mx(x)
        b, sb = ofp4.quantize_mx(w)
        ta = tb = None
        ofp4.gemm_ref(ofp4.MX, a, sa, b, sb)
        ofp4.dequantize_mx(a, sa)
    else:
        a, sa, ta = ofp4.quantize_nv(x)
        b, sb, tb = ofp4.quantize_nv(w)
        ofp4.gemm_ref(ofp4.NV, a, sa, b, sb, ta, tb)
        ofp4.dequantize_nv(a, sa, ta)
    dt = time.perf_counter() - t0
    threads = blas_threads()
    flops = 2.0 * x_rows * w_rows * wl.K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": host_cores(), "kind": "oracle",
            "blas_threads": int(threads), "quantize_threads": 1,
            "sample": f"{x_rows} of {wl.M} rows of X and {w_rows} of {wl.N} rows of W: oracle FP4 quantize of "
                      f"both, fp64 GEMM of the sample (numpy BLAS threads={threads}), dequantize of X; "
                      f"{dt:.2f} s"}


def fp4_gemm_bytes(wl) -> int:
    """Algorithmic bytes of one FP4 GEMM: both operands' codes (half a byte
    per element) and block scales (one byte per 32 (MX) or 16 (NV) elements)
    read once, the bf16 output written once."""
    blk = 32 if wl.fp4_kind == workloads.FP4_MX else 16
    return (wl.M + wl.N) * (wl.K // 2 + wl.K // blk) + wl.M * wl.N * 2


def bench_fp4(args, wl) -> int:
    import torch
    import block_scaled_precision_x128_amd as fb

    fb.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    M, N, K, kind = wl.M, wl.N, wl.K, wl.fp4_kind
    xs_np, ws_np = workloads.make_inputs(wl)
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    x0, w0 = to_dev(xs_np), to_dev(ws_np)
    del xs_np, ws_np
    blk = fb.fp4_block(kind)
    qbytes = lambda rows: rows * K * 2 + rows * K // 2 + rows * (K // blk)
    big = [b for b in (qbytes(M), qbytes(N), fp4_gemm_bytes(wl)) if b >= 8e6]
    R = args.sets or (int(min(32, max(2, np.ceil(ROTATION_BYTES / min(big))))) if big else 2)
    sets = []
    for r in range(R):
        x = x0 if r == 0 else x0.clone()
        w = w0 if r == 0 else w0.clone()
        xq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
        xs = torch.empty((M, K // blk), dtype=torch.uint8, device=dev)
        wsc = torch.empty((N, K // blk), dtype=torch.uint8, device=dev)
        xt = torch.empty(1, dtype=torch.float32, device=dev) if kind == fb.FP4_NV else None
        wt = torch.empty(1, dtype=torch.float32, device=dev) if kind == fb.FP4_NV else None
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        xr = torch.empty_like(x)
        sets.append((x, w, xq, wq, xs, wsc, xt, wt, out, xr))
    wsx = torch.empty(max(1, fb.fp4_quantize_workspace_bytes(M, K, kind)), dtype=torch.uint8, device=dev)
    wsw = torch.empty(max(1, fb.fp4_quantize_workspace_bytes(N, K, kind)), dtype=torch.uint8, device=dev)

    qx = lambda st, s=None: fb.fp4_quantize(st[0], kind, q=st[2], block_scales=st[4], tensor_scale=st[6],
                                            workspace=wsx, stream=s)
    qw = lambda st, s=None: fb.fp4_quantize(st[1], kind, q=st[3], block_scales=st[5], tensor_scale=st[7],
                                            workspace=wsw, stream=s)
    gm = lambda st, s=None: fb.fp4_gemm_blockscaled(st[2], st[4], st[6], st[3], st[5], st[7], kind, fb.DT_BF16,
                                                    out=st[8], stream=s)
    dq = lambda st, s=None: fb.fp4_dequantize(st[2], st[4], st[6], kind, fb.DT_BF16, y=st[9], stream=s)
    # Decode shapes (M <= 64) quantize the weights once, in setup, as a model's
    # weights are; the step streams them through the skinny kernel.
    decode = M <= 64
    for st in sets:
        qx(st)
        qw(st)
    torch.cuda.synchronize()

    def step(i, s):
        st = sets[i % R]
        qx(st, s)
        if not decode:
            qw(st, s)
        gm(st, s)
        dq(st, s)

    for i in range(args.warmup):
        step(i, stream)
    torch.cuda.synchronize()
    timer = Timer(torch, preroll_ms=args.preroll_ms)
    wall0 = time.perf_counter()
    step_batches = timer.batches(step, args.steps)
    wall = time.perf_counter() - wall0
    ms_step = median(step_batches)
    at = lambda f: (lambda i, s: f(sets[i % R], s))
    qx_ms, qw_ms, gm_ms, dq_ms = (median(timer.batches(at(f), args.steps)) for f in (qx, qw, gm, dq))
    flops = 2.0 * M * N * K
    gemm_tflops = flops / (gm_ms * 1e-3) / 1e12
    traffic = read_traffic(wl.name, "fp32")
    # MXFP4 runs on the FP4 matrix cores (exact block sums); NVFP4 expands its
    # codes times microscales to fp16 and runs on the fp16 ones.  Decode shapes
    # are bound by streaming the weights: algorithmic bytes against HBM.
    peak = PEAK_FP4_TFLOPS if kind == fb.FP4_MX else PEAK_BF16_TFLOPS
    gemm_gbs = fp4_gemm_bytes(wl) / (gm_ms * 1e-3) / 1e9
    if decode:
        roofline = {"bound": "hbm", "achieved": round(gemm_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gemm_gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        roofline = {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(gemm_tflops / peak, 4), "traffic": traffic}
    result = {
        "metric": "block-scaled FP4 GEMM TFLOP/s (exact products, fp32 sums); quantize GB/s",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4",
        "data": "synthetic (seeded; bf16 activations ~N(0,1) with outlier channels, weights ~N(0,0.02))",
        "config": {"workload": f"{wl.name}: M={M} N={N} K={K}, E2M1 operands, "
                               + ("MXFP4 (UE8M0 per 32)" if kind == fb.FP4_MX else
                                  "NVFP4 (E4M3 per 16 + fp32 tensor scale)") + ", bf16 out",
                   "step": ("quantize X + GEMM + dequantize X (W quantized in setup)" if decode else
                            "quantize X + quantize W + GEMM + dequantize X"),
                   "rotated_input_sets": R,
                   "accumulation": ("FP4 matrix cores with UE8M0 block scales: exact 32-element block sums, "
                                    "fp32 sums" if kind == fb.FP4_MX else
                                    "codes times E4M3 microscales expanded exactly to fp16, fp16 matrix cores, "
                                    "fp32 sums")},
        "roofline": roofline,
        "kernels": {"gemm_ms": round(gm_ms, 4), "gemm_tflops": round(gemm_tflops, 1),
                    "gemm_algorithmic_gbs": round(gemm_gbs, 1), "quantize_w_in_step": not decode,
                    "quantize_x_ms": round(qx_ms, 4), "quantize_x_gbs": round(qbytes(M) / (qx_ms * 1e-3) / 1e9, 1),
                    "quantize_w_ms": round(qw_ms, 4), "quantize_w_gbs": round(qbytes(N) / (qw_ms * 1e-3) / 1e9, 1),
                    "dequantize_x_ms": round(dq_ms, 4),
                    "dequantize_x_gbs": round((M * K // 2 + M * (K // blk) + M * K * 2) / (dq_ms * 1e-3) / 1e9, 1)},
        "step_batches_ms": [round(x, 4) for x in step_batches],
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_ceilings:
        # the HBM-bound kernels against a read or copy of their own byte volume
        sized = SizedCeilings(torch, fb, timer, args.steps)
        kern = result["kernels"]
        items = [("quantize_x", qbytes(M), "copy"), ("quantize_w", qbytes(N), "copy"),
                 ("dequantize_x", M * K // 2 + M * (K // blk) + M * K * 2, "copy")]
        for key, nbytes, how in items:
            g = sized.gbs(how, nbytes)
            kern[f"{key}_ceiling_gbs"] = round(g, 1)
            kern[f"{key}_frac_ceiling"] = round(kern[f"{key}_gbs"] / g, 4)
        if decode:
            g = sized.gbs("read", fp4_gemm_bytes(wl))
            kern["gemm_ceiling_gbs"] = round(g, 1)
            kern["gemm_frac_ceiling"] = round(gemm_gbs / g, 4)
        del sized
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = fp4_cpu_baseline(wl, min(1024, M), 4096)
    print(json.dumps(result), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3_deepseek_block",
                    choices=workloads.CONFIG_ORDER + list(workloads.KV_CONFIGS) + list(workloads.FP4_CONFIGS))
    ap.add_argument("--sets", type=int, default=0, help="rotated input sets (0 = enough for 1 GB)")
    ap.add_argument("--accum", choices=["fp32", "native"], default="fp32",
                    help="GEMM accumulation: exact products with fp32 sums (default) or the FP8 "
                         "instructions' own accumulation")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="time only the selected workload (the default c3 run also times c1, c2, c4, c5)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the MFMA/read/copy ceiling probes")
    ap.add_argument("--cpu-sample-rows", type=int, default=4096)
    ap.add_argument("--kv-cpu-sample-tokens", type=int, default=16384)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 256 MiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--summarize-trace", metavar="DIR", help="print a rocprofv3 kernel-trace summary and exit")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                                "COPY_WRITE_CSV"),
                    help="print the calibrated HBM traffic of the GEMM kernel and exit")
    ap.add_argument("--kernel-match", default=GEMM_KERNEL_RE,
                    help="kernel-name regular expression for --summarize-traffic")
    ap.add_argument("--traffic-sources", choices=["gemm", "kv"], default="gemm",
                    help="which kernel sources the --summarize-traffic hash covers")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="print per-kernel means of the counters in these rocprofv3 --pmc CSV files and exit")
    ap.add_argument("--preroll-ms", type=float, default=60.0,
                    help="untimed back-to-back work before each timed batch (clock ramp)")
    ap.add_argument("--profile-gemm", type=int, default=0, metavar="N",
                    help="only run the workload's GEMM N times on its bench inputs (for rocprofv3 --pmc runs)")
    ap.add_argument("--min-grid", type=int, default=0,
                    help="--summarize-traffic: only dispatches of at least this many threads")
    args = ap.parse_args(argv)

    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return 0
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters, args.kernel_match))
        return 0
    if args.summarize_traffic:
        print(summarize_traffic(*args.summarize_traffic, args.kernel_match, COPY_PROBE_BYTES,
                                KV_SOURCES if args.traffic_sources == "kv" else GEMM_SOURCES, args.min_grid))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (each GPU would run the same "
              "kernels on its own shard); run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import block_scaled_precision_x128_amd as fb

    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        return 1
    fb.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    if args.copy_probe:
        n = COPY_PROBE_BYTES
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n}))
        return 0

    if args.workload in workloads.KV_CONFIGS:
        return bench_kv(args, workloads.KV_CONFIGS[args.workload])
    if args.workload in workloads.FP4_CONFIGS:
        return bench_fp4(args, workloads.FP4_CONFIGS[args.workload])

    wl = workloads.CONFIGS[args.workload]
    accum = fb.ACCUM_NATIVE if args.accum == "native" else fb.ACCUM_FP32
    if args.profile_gemm:
        return profile_gemm(torch, fb, wl, accum, args.profile_gemm)
    timer = Timer(torch, preroll_ms=args.preroll_ms)
    head = fp8_workload(torch, fb, timer, wl, args, accum, headline=True)
    result = head.pop("result")

    # The other workloads of the path, GPU kernels only (no CPU leg): each
    # config's quantize, GEMM and dequantize, timed the same way.
    if args.workload == "c3_deepseek_block" and not args.no_other_configs:
        others = {}
        for name in workloads.CONFIG_ORDER:
            if name == wl.name:
                continue
            others[name] = fp8_workload(torch, fb, timer, workloads.CONFIGS[name], args, accum, headline=False)
            torch.cuda.empty_cache()
        result["configs"] = others
    if not args.no_ceilings:
        result["ceilings"] = measure_ceilings(torch, fb, timer, args.steps)
        # HBM-bound kernels against a read or copy of their own byte volume
        sized = SizedCeilings(torch, fb, timer, args.steps)
        sized.annotate(result["kernels"], wl)
        for name, kern in result.get("configs", {}).items():
            sized.annotate(kern, workloads.CONFIGS[name])
        result["ceilings"]["sized_note"] = ("<kernel>_ceiling_gbs: the read probe (decode GEMM) or the copy probe "
                                            "(quantize, dequantize; half the bytes read, half written) moving the "
                                            "kernel's own byte volume, over disjoint slices of 1 GiB buffers")
        del sized
        torch.cuda.empty_cache()
        torch.cuda.empty_cache()
    result["gpu_clocks"] = gpu_clocks()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, min(args.cpu_sample_rows, wl.M))
    print(json.dumps(result), flush=True)
    return 0


def profile_gemm(torch, fb, wl, accum, n: int) -> int:
    """The workload's GEMM alone, n launches on the bench's inputs (quantized
    by the library), for counter runs."""
    dev = torch.device("cuda:0")
    xs_np, ws_np = workloads.make_inputs(wl)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    xq, sx = fb.fp8_quantize(to_dev(xs_np), wl.x_fmt, wl.x_gran)
    wq, sw = fb.fp8_quantize(to_dev(ws_np), wl.w_fmt, wl.w_gran)
    out = torch.empty((wl.M, wl.N), dtype=torch.bfloat16 if wl.out_dtype == fb.DT_BF16 else torch.float32,
                      device=dev)
    for _ in range(n):
        fb.fp8_gemm_blockscaled(xq, wl.x_fmt, wl.x_gran, sx, wq, wl.w_fmt, wl.w_gran, sw, wl.out_dtype, out=out,
                                accum=accum)
    torch.cuda.synchronize()
    print(json.dumps({"profile_gemm": wl.name, "launches": n, "accum": "native" if accum == fb.ACCUM_NATIVE
                      else "fp32"}), flush=True)
    return 0


def fp8_workload(torch, fb, timer, wl, args, accum, headline: bool):
    """Time one FP8 workload.  With headline=True: the whole step (quantize X,
    quantize W unless W is a decode shape's pre-quantized weight, GEMM,
    dequantize X) over exactly --steps steps per batch, then each kernel on its
    own, and the bench JSON line; otherwise only the per-kernel figures."""
    dev = torch.device("cuda:0")
    M, N, K = wl.M, wl.N, wl.K
    xs_np, ws_np = workloads.make_inputs(wl)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    x0, w0 = to_dev(xs_np), to_dev(ws_np)
    del xs_np, ws_np
    in_b = 2 if wl.in_dtype == workloads.DT_BF16 else 4
    R = args.sets or rotation_sets(wl)
    sets = []
    for r in range(R):
        x = x0 if r == 0 else x0.clone()
        w = w0 if r == 0 else w0.clone()
        xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
        wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
        sdt = lambda g: torch.uint8 if g == fb.GRAN_MX32 else torch.float32
        sx = torch.empty(fb.scale_shape(wl.x_gran, M, K), dtype=sdt(wl.x_gran), device=dev)
        sw = torch.empty(fb.scale_shape(wl.w_gran, N, K), dtype=sdt(wl.w_gran), device=dev)
        out = torch.empty((M, N), dtype=torch.bfloat16 if wl.out_dtype == fb.DT_BF16 else torch.float32, device=dev)
        xr = torch.empty_like(x)   # dequantized X
        sets.append((x, w, xq, wq, sx, sw, out, xr))
    wsx = torch.empty(max(1, fb.fp8_quantize_workspace_bytes(M, K, wl.x_gran)), dtype=torch.uint8, device=dev)
    wsw = torch.empty(max(1, fb.fp8_quantize_workspace_bytes(N, K, wl.w_gran)), dtype=torch.uint8, device=dev)
    # Decode (M <= 64): the weights are quantized once, in setup, as a model's are.
    w_in_step = wl.M > 64
    for st in sets:
        fb.fp8_quantize(st[0], wl.x_fmt, wl.x_gran, q=st[2], scales=st[4], workspace=wsx)
        fb.fp8_quantize(st[1], wl.w_fmt, wl.w_gran, q=st[3], scales=st[5], workspace=wsw)
    torch.cuda.synchronize()

    qx = lambda st, s: fb.fp8_quantize(st[0], wl.x_fmt, wl.x_gran, q=st[2], scales=st[4], workspace=wsx, stream=s)
    qw = lambda st, s: fb.fp8_quantize(st[1], wl.w_fmt, wl.w_gran, q=st[3], scales=st[5], workspace=wsw, stream=s)
    gm = lambda st, s: fb.fp8_gemm_blockscaled(st[2], wl.x_fmt, wl.x_gran, st[4], st[3], wl.w_fmt, wl.w_gran, st[5],
                                               wl.out_dtype, out=st[6], accum=accum, stream=s)
    dq = lambda st, s: fb.fp8_dequantize(st[2], st[4], wl.x_fmt, wl.x_gran, wl.in_dtype, y=st[7], stream=s)

    def step(i, s):
        st = sets[i % R]
        qx(st, s)
        if w_in_step:
            qw(st, s)
        gm(st, s)
        dq(st, s)

    K_steps = args.steps
    rot = lambda f: (lambda i, s: f(sets[i % R], s))
    res = {}
    if headline:
        for i in range(args.warmup):
            step(i, torch.cuda.current_stream())
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        step_batches = timer.batches(step, K_steps)
        wall = time.perf_counter() - wall0
    kms = {}
    for name, f in (("quantize_x", qx), ("quantize_w", qw), ("gemm", gm), ("dequantize_x", dq)):
        kms[name] = timer.batches(rot(f), K_steps)
    med = {k: median(v) for k, v in kms.items()}

    flops = 2.0 * M * N * K
    gemm_tflops = flops / (med["gemm"] * 1e-3) / 1e12
    qx_gbs = quant_bytes(wl, "x") / (med["quantize_x"] * 1e-3) / 1e9
    qw_gbs = quant_bytes(wl, "w") / (med["quantize_w"] * 1e-3) / 1e9
    dq_gbs = dequant_bytes(wl) / (med["dequantize_x"] * 1e-3) / 1e9
    gemm_hbm_gbs = gemm_bytes(wl) / (med["gemm"] * 1e-3) / 1e9
    kern = {
        "gemm_ms": round(med["gemm"], 4), "gemm_tflops": round(gemm_tflops, 1),
        "gemm_frac_fp8_peak": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
        "gemm_frac_bf16_peak": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
        "gemm_algorithmic_gbs": round(gemm_hbm_gbs, 1),
        "gemm_frac_hbm": round(gemm_hbm_gbs / PEAK_HBM_GBS, 4),
        "quantize_x_ms": round(med["quantize_x"], 4), "quantize_x_gbs": round(qx_gbs, 1),
        "quantize_x_frac_hbm": round(qx_gbs / PEAK_HBM_GBS, 4),
        "quantize_w_ms": round(med["quantize_w"], 4), "quantize_w_gbs": round(qw_gbs, 1),
        "quantize_w_frac_hbm": round(qw_gbs / PEAK_HBM_GBS, 4),
        "quantize_w_in_step": w_in_step,
        "dequantize_x_ms": round(med["dequantize_x"], 4), "dequantize_x_gbs": round(dq_gbs, 1),
        "dequantize_x_frac_hbm": round(dq_gbs / PEAK_HBM_GBS, 4),
        "batches_ms": {k: [round(x, 4) for x in v] for k, v in kms.items()},
        "shape": f"M={M} N={N} K={K}", "rotated_input_sets": R,
    }
    if not headline:
        return kern

    # Delayed scaling of X as a whole tensor (scale from an amax history of
    # 16 iterations): one read of the input, against the two reads of
    # current per-tensor scaling.
    hist = torch.zeros(16, dtype=torch.float32, device=dev)
    dsc = torch.empty(1, dtype=torch.float32, device=dev)
    wsd = torch.empty(max(1, fb.fp8_quantize_workspace_bytes(M, K, fb.GRAN_TENSOR)), dtype=torch.uint8, device=dev)
    delayed = lambda i, s: fb.fp8_quantize_delayed(sets[i % R][0], wl.x_fmt, hist, i % 16, q=sets[i % R][2],
                                                   scale=dsc, workspace=wsd, stream=s)
    qd_ms = median(timer.batches(delayed, K_steps))
    qd_bytes = M * K * (in_b + 1) + 8
    qd_gbs = qd_bytes / (qd_ms * 1e-3) / 1e9
    kern.update({"quantize_x_delayed_ms": round(qd_ms, 4), "quantize_x_delayed_gbs": round(qd_gbs, 1),
                 "quantize_x_delayed_frac_hbm": round(qd_gbs / PEAK_HBM_GBS, 4)})

    # The next row of the path: the GEMM with its output quantized in the
    # epilogue (E4M3 codes + 1x128 tile scales), against the GEMM followed by
    # a separate quantize of its output.
    fused = None
    if wl.M > 64 and N % 128 == 0:
        oq = torch.empty((M, N), dtype=torch.uint8, device=dev)
        osc = torch.empty((M, N // 128), dtype=torch.float32, device=dev)
        fq = lambda st, s: fb.fp8_gemm_blockscaled_quant(st[2], wl.x_fmt, wl.x_gran, st[4], st[3], wl.w_fmt,
                                                         wl.w_gran, st[5], fb.E4M3, codes=oq, scales=osc,
                                                         accum=accum, stream=s)
        qo = lambda st, s: fb.fp8_quantize(st[6], fb.E4M3, fb.GRAN_TILE_1x128, q=oq, scales=osc, stream=s)
        fq_ms = median(timer.batches(rot(fq), K_steps))
        qo_ms = median(timer.batches(rot(qo), K_steps))
        fused = {"gemm_quantized_out_ms": round(fq_ms, 4), "gemm_then_quantize_ms": round(med["gemm"] + qo_ms, 4),
                 "quantize_out_ms": round(qo_ms, 4)}
    kern["fused_epilogue_quantize"] = fused

    ms_step = median(step_batches)
    value = flops / (ms_step * 1e-3) / 1e12
    skinny = wl.M <= 64
    traffic = read_traffic(wl.name, args.accum)
    if skinny:
        roof = {"bound": "hbm", "achieved": round(gemm_hbm_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gemm_hbm_gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        # Priced against the dense fp8 matrix-core peak, the metric's own
        # denominator.  The exact default multiplies on the bf16 matrix cores
        # (half that rate), so its fraction of the bf16 peak is in `kernels`.
        roof = {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4), "traffic": traffic}
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic (seeded; bf16 activations ~N(0,1) with outlier channels, weights ~N(0,0.02))",
        "config": {"workload": f"{wl.name}: M={M} N={N} K={K}, X 1x128 tiles, W 128x128 blocks, "
                               f"E4M3, fp32 scales, bf16 out" if wl.name == "c3_deepseek_block" else
                               f"{wl.name}: M={M} N={N} K={K}",
                   "step": "quantize X + quantize W + GEMM + dequantize X" if w_in_step else
                           "quantize X + GEMM + dequantize X (W quantized once in setup)",
                   "rotated_input_sets": R,
                   "timing": (f"{args.warmup} eager warm-up steps; then 5 batches of exactly {K_steps} steps, each "
                              f"queued behind a spin and an untimed pre-roll of >= {timer.preroll_ms:.0f} ms of the "
                              f"same steps, bracketed by HIP events and device synchronizes; ms_per_step is the "
                              f"median batch (step_batches_ms lists all 5); each kernel is timed the same way, "
                              f"{K_steps} launches per batch"),
                   "accumulation": ("fp8 MFMA, the instruction's own accumulation" if accum == fb.ACCUM_NATIVE else
                                    "fp8 codes expanded exactly to bf16, bf16 MFMA, fp32 accumulation")},
        "roofline": roof,
        "kernels": kern,
        "step_batches_ms": [round(x, 4) for x in step_batches],
        "wall_s_timed": round(wall, 4),
    }
    return {"result": result}


if __name__ == "__main__":
    sys.exit(main())
