"""Host logic of bench.py (no GPU): the one-GPU refusal, the algorithmic work it prices
launches against, and the conversion of rocprofv3 counter CSVs into bytes and flops."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_ce_algorithmic_bytes_at_the_large_vocabulary_workload():
    # 16384 rows, V = 128256, 819 ignored: the forward reads the 15565 labelled rows, the
    # in-place backward reads them again and writes all 16384 rows
    fwd, bwd = bench.ce_algorithmic_bytes(16384, 128256, 15565)
    assert fwd == 3_992_609_280
    assert bwd == 8_195_301_888
    assert fwd + bwd == 12_187_911_168


def test_flce_launch_pricing_at_the_llama3_head():
    w = workloads.WORKLOADS["flce_8192x4096x128256"]
    n, h, v = w.n, w.h, w.v
    # paired chunks: four grad_weight launches of K = 2048; probabilities and hidden rows
    # once, the accumulator written by the first launch and read and written by the other
    # three: (4 + 3 * 8) / 4 = 7 bytes per element
    k = 2048
    assert bench.gemm_bytes("flce_gemm_grad_weight", w, 4) == 2 * k * v + 2 * k * h + 7 * v * h
    assert bench.gemm_bytes("flce_gemm_grad_hidden", w, 8) == 2 * 1024 * v + 2 * v * h + 2 * 1024 * h
    # transposed probabilities: five grad_weight launches over vocabulary ranges, K = n; all
    # of Pᵀ once, the hidden rows once per launch, grad_weight written once
    assert bench.gemm_bytes("flce_gemm_grad_weight", w, 5, transposed=True) == \
        (2 * n * v + 5 * 2 * n * h + 4 * v * h) / 5
    assert bench.gemm_bytes("flce_gemm_grad_hidden", w, 1, transposed=True) == \
        2 * n * v + 2 * v * h + 2 * n * h
    # the logits product is the same in both
    for t in (False, True):
        assert bench.gemm_bytes("flce_gemm_logits", w, 8, transposed=t) == \
            2 * v * h + 2 * 1024 * h + 2 * 1024 * v
    assert bench.gemm_bytes("flce_gemm_logits", w, 8, stored_slice=False) == 2 * v * h + 2 * 1024 * h


def test_roofline_takes_the_higher_floor():
    # grad_weight at the Llama3 head: 2.15e12 flop and 4.22e9 B per launch, 510 flop/B,
    # above the 312.5 flop/B ridge: MFMA-bound
    w = workloads.WORKLOADS["flce_8192x4096x128256"]
    flops = 2.0 * 2048 * w.h * w.v
    nbytes = bench.gemm_bytes("flce_gemm_grad_weight", w, 4)
    r = bench.gemm_roofline("flce_gemm_grad_weight", flops, nbytes, 2.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(flops / 2e-3 / 1e12, rel=1e-3)
    assert r["hbm"]["algorithmic_bytes"] == int(nbytes)
    # the same launch with a tenth of the flops is HBM-bound
    r = bench.gemm_roofline("flce_gemm_grad_weight", flops / 10, nbytes, 2.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            wr.writerow(r)


def test_traffic_is_scaled_by_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path / "profiles"))
    gib_kib = (1 << 30) / 1024.0
    # the copy reads 1 GiB and writes 1 GiB; FETCH_SIZE sees half of its reads
    fetch = [(1, "neg_kernel_cuda", "FETCH_SIZE", gib_kib / 2),
             (2, "gemm_pipe_kernel<..., EpiGradWeight>", "FETCH_SIZE", 1000.0),
             (3, "gemm_pipe_kernel<..., EpiGradWeight>", "FETCH_SIZE", 3000.0)]
    write = [(1, "neg_kernel_cuda", "WRITE_SIZE", gib_kib),
             (2, "gemm_pipe_kernel<..., EpiGradWeight>", "WRITE_SIZE", 500.0),
             (3, "gemm_pipe_kernel<..., EpiGradWeight>", "WRITE_SIZE", 500.0)]
    _write_counters(tmp_path / "f", fetch)
    _write_counters(tmp_path / "w", write)
    bench.record_traffic("flce_8192x4096x128256", str(tmp_path / "f"), str(tmp_path / "w"))
    rec = json.load(open(tmp_path / "profiles" / "traffic.json"))[
        "flce_gemm_grad_weight@flce_8192x4096x128256"]
    assert rec["read_bytes"] == 2 * 2000 * 1024  # mean 2000 KiB per dispatch, factor 2
    assert rec["write_bytes"] == 500 * 1024
    assert bench.stored_traffic("flce_gemm_grad_weight", "flce_8192x4096x128256") == \
        rec["read_bytes"] + rec["write_bytes"]
    # counters recorded for other sources are not used
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 16)
    assert bench.stored_traffic("flce_gemm_grad_weight", "flce_8192x4096x128256") is None


def test_mfma_counters_give_flops_busy_fraction_and_clock(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path / "profiles"))
    name = "gemm_pipe_kernel<..., EpiLogits16>"
    mops = 2.0 * 1024 * 4096 * 128256 / 512  # one launch of the logits product
    active = 8 * 2.0e6  # GRBM_GUI_ACTIVE summed over the 8 XCDs: 2e6 cycles each
    busy = 0.5 * 2.0e6 * 1024  # half of the 1024 SIMDs' cycles
    rows = []
    for d in (1, 2):
        rows += [(d, name, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops),
                 (d, name, "SQ_VALU_MFMA_BUSY_CYCLES", busy), (d, name, "GRBM_GUI_ACTIVE", active)]
    _write_counters(tmp_path / "p", rows)
    os.makedirs(tmp_path / "t")
    with open(tmp_path / "t" / "run_kernel_trace.csv", "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for s in (0, 5_000_000):
            wr.writerow([name, s, s + 1_000_000])  # 1 ms each
    bench.record_mfma("flce_8192x4096x128256", str(tmp_path / "p"), str(tmp_path / "t"))
    got = bench.stored_mfma("flce_gemm_logits", "flce_8192x4096x128256")
    assert got["flops_per_launch"] == pytest.approx(2.0 * 1024 * 4096 * 128256)
    assert got["mfma_busy_frac"] == pytest.approx(0.5)
    assert got["clock_ghz"] == pytest.approx(2.0)
