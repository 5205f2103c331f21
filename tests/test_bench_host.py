"""Host-side checks of bench.py: the one-GPU contract, the algorithmic byte
counts its roofline uses, and the counter-summary arithmetic (no GPU needed)."""

import csv
import os

import pytest

import bench
import workloads


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.parametrize("name,operand,want", [
    # input read once (2 B bf16) + one code byte per element + the scales
    ("c3_deepseek_block", "x", 4096 * 7168 * 3 + 4096 * 56 * 4),
    ("c3_deepseek_block", "w", 7168 * 7168 * 3 + 56 * 56 * 4),
    ("c2_per_token_channel", "x", 2048 * 4096 * 3 + 2048 * 4),
    ("c5_mxfp8_mix", "w", 8192 * 8192 * 5 + 8192 * 256),
])
def test_quantize_bytes(name, operand, want):
    assert bench.quant_bytes(workloads.CONFIGS[name], operand) == want


def test_gemm_and_dequantize_bytes():
    c4 = workloads.CONFIGS["c4_decode_skinny"]
    # W codes + W block scales + X codes + X tile scales + bf16 out
    assert bench.gemm_bytes(c4) == 132120576 + 32256 + 114688 + 3584 + 589824
    c3 = workloads.CONFIGS["c3_deepseek_block"]
    assert bench.dequant_bytes(c3) == 4096 * 7168 * 3 + 4096 * 56 * 4


def test_fp4_gemm_bytes():
    dec = workloads.FP4_CONFIGS["fp4_mx_decode_16x18432x7168"]
    # codes (K/2 bytes a row) + UE8M0 scales (K/32) of X and W, bf16 out
    assert bench.fp4_gemm_bytes(dec) == (16 + 18432) * (3584 + 224) + 16 * 18432 * 2 == 70839808
    nvd = workloads.FP4_CONFIGS["fp4_nv_decode_16x18432x7168"]
    # NV microscales: one E4M3 byte per 16 elements (the tensor scales are 8 bytes, not counted)
    assert bench.fp4_gemm_bytes(nvd) == (16 + 18432) * (3584 + 448) + 16 * 18432 * 2
    nv = workloads.FP4_CONFIGS["fp4_nv_4096x7168x7168"]
    assert bench.fp4_gemm_bytes(nv) == (4096 + 7168) * (3584 + 448) + 4096 * 7168 * 2


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for i, (name, ctr, val) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": ctr, "Counter_Value": val})


def test_traffic_summary_calibration(tmp_path):
    kib = bench.COPY_PROBE_BYTES / 1024
    big, split, quant = ("k_gemm_tiled_256x256<0, 0, 1, 1, 0>(args)", "k_gemm_tiled_256x192<0, 0, 1, 1, 0>(args)",
                         "k_gemm_tiled_256x256<0, 0, 1, 2, 0>(args)")
    _csv(tmp_path / "f.csv", [(big, "FETCH_SIZE", 100.0), (split, "FETCH_SIZE", 30.0), (big, "FETCH_SIZE", 300.0),
                              (split, "FETCH_SIZE", 10.0), (quant, "FETCH_SIZE", 7e6), ("other", "FETCH_SIZE", 9e9)])
    _csv(tmp_path / "w.csv", [(big, "WRITE_SIZE", 50.0), (split, "WRITE_SIZE", 5.0), (big, "WRITE_SIZE", 50.0),
                              (split, "WRITE_SIZE", 15.0), (quant, "WRITE_SIZE", 3e6)])
    _csv(tmp_path / "cf.csv", [("fill", "FETCH_SIZE", 1.0), ("copy", "FETCH_SIZE", kib / 2)])
    _csv(tmp_path / "cw.csv", [("copy", "WRITE_SIZE", kib)])
    text = bench.summarize_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                                   str(tmp_path / "cw.csv"), bench.GEMM_KERNEL_RE, bench.COPY_PROBE_BYTES)
    kv = dict(line.split(":", 1) for line in text.splitlines() if not line.startswith(" "))
    # fetch counter reads half the copy: factor 2.  One launch = one dispatch of
    # each tile shape: fetch (200 + 20) KiB -> 440 KiB; writes 50 + 10 KiB.  The
    # quantized-output kernel and unrelated kernels are not part of it.
    assert float(kv["fetch_factor"].split()[0]) == pytest.approx(2.0)
    assert float(kv["traffic_bytes_per_launch"]) == pytest.approx((440 + 60) * 1024)
    assert kv["source_sha256"].strip() == bench.gemm_source_hash()


def test_stored_traffic_needs_matching_sources(tmp_path, monkeypatch):
    path = tmp_path / "t.txt"
    monkeypatch.setattr(bench, "traffic_path", lambda wl, acc: str(path))
    assert bench.read_traffic("c3_deepseek_block", "fp32") is None
    path.write_text("# header\ntraffic_bytes_per_launch: 1234\nsource_sha256: " + "0" * 64 + "\n")
    assert bench.read_traffic("c3_deepseek_block", "fp32") is None
    path.write_text("traffic_bytes_per_launch: 1234\nsource_sha256: " + bench.gemm_source_hash() + "\n")
    assert bench.read_traffic("c3_deepseek_block", "fp32") == 1234


def test_committed_profiles_parse():
    """Every stored traffic summary carries the fields bench.py reads."""
    pdir = os.path.join(bench.ROOT, "profiles")
    files = [f for f in os.listdir(pdir) if f.startswith("traffic_")]
    assert files
    for f in files:
        text = open(os.path.join(pdir, f)).read()
        assert "traffic_bytes_per_launch:" in text and "source_sha256:" in text
