"""Host-side logic of bench.py: counter-run summary, traffic scaling, multi-GPU refusal."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from state_space_sequence_cumsum_amd.inputs import WORKLOADS  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_run(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": v})


def test_summarize_pmc_scales_by_copy(tmp_path, monkeypatch):
    w = WORKLOADS["fp32_b1_L256_H4_P64_N64_Q64"]
    monkeypatch.setattr(bench, "traffic_file", lambda w_: str(tmp_path / "traffic.json"))
    copy_mib = 4
    # the copy reads half its size in FETCH_SIZE and all of it in WRITE_SIZE
    _write_run(tmp_path / "f", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", copy_mib * 512.0),
                                              ("__amd_rocclr_copyBuffer", 1.0),
                                              ("void ssd::chunk_out_kernel<float, 64>(...)", 100.0),
                                              ("void ssd::chunk_out_kernel<float, 64>(...)", 300.0)])
    _write_run(tmp_path / "w", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", copy_mib * 1024.0),
                                              ("void ssd::chunk_out_kernel<float, 64>(...)", 50.0)])
    bench.summarize_pmc(w, str(tmp_path / "f"), str(tmp_path / "w"), copy_mib)
    out = json.load(open(tmp_path / "traffic.json"))
    assert out["fetch_scale"] == pytest.approx(2.0)
    assert out["write_scale"] == pytest.approx(1.0)
    k = out["kernels"]["chunk_out"]
    assert k["fetch_kib"] == pytest.approx(200.0) and k["dispatches"] == 2
    assert k["traffic_bytes"] == pytest.approx((200.0 * 2.0 + 50.0) * 1024.0)
    assert out["source_hash"] == bench.source_hash()


def test_summarize_pmc_needs_copy(tmp_path, monkeypatch):
    w = WORKLOADS["fp32_b1_L256_H4_P64_N64_Q64"]
    monkeypatch.setattr(bench, "traffic_file", lambda w_: str(tmp_path / "traffic.json"))
    _write_run(tmp_path / "f", "FETCH_SIZE", [("chunk_out_kernel", 1.0)])
    _write_run(tmp_path / "w", "WRITE_SIZE", [("chunk_out_kernel", 1.0)])
    with pytest.raises(SystemExit):
        bench.summarize_pmc(w, str(tmp_path / "f"), str(tmp_path / "w"), 4)


def test_algorithmic_headline_bytes():
    w = WORKLOADS["bf16_b1_L16384_H32_P64_N256_Q256"]
    a = bench.algorithmic(w)
    th = 16384 * 32
    # chunk out: x and y (2 B each, 64 wide), G2 and dtT, B and C once per group, S read
    assert a["chunk_out"]["bytes"] == th * (2 * 2 * 64 + 8 + 2 * 2 * 256 / 32 + 2 * 64 * 256 / 256)
    assert a["state_pass"]["flops"] == th * 2 * 256 * 64


def test_multi_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_percentile_nearest_rank():
    v = [float(i) for i in range(1, 11)]
    assert bench.pct(v, 10) == 2.0 and bench.pct(v, 50) in (5.0, 6.0) and bench.pct(v, 90) == 9.0
    assert bench.pct([3.0], 90) == 3.0
    assert bench.pct([5.0, 1.0, 3.0], 0) == 1.0 and bench.pct([5.0, 1.0, 3.0], 100) == 5.0


def test_step_algorithmic_bytes():
    # batch 128 of the headline heads: fp32 state read and written dominates
    w = WORKLOADS["bf16_b1_L16384_H32_P64_N256_Q256"]
    a = bench.step_algorithmic(w, 128)
    state = 128 * 32 * 64 * 256 * 4 * 2
    io = 128 * 32 * (2 * 2 * 64 + 2) + 128 * 1 * 2 * 2 * 256 + 8 * 32
    assert a["bytes"] == state + io


def test_sweep_grid_covers_the_pages_range():
    assert bench.SWEEP_TOKENS[0] == 1024 and bench.SWEEP_TOKENS[-1] == 262144
    assert bench.SWEEP_STATES == [64, 128, 256, 512]
    assert bench.SWEEP_BASE in WORKLOADS
