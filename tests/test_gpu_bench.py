"""bench.py on the GPU, in-process: the one JSON line it prints keeps the benchmark contract
(metric, value, unit, steps, timing, roofline and cpu_baseline objects), on small workloads
with few steps, in the default, --autotune and --step modes."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import state_space_sequence_cumsum_amd as ssd  # noqa: E402

pytestmark = pytest.mark.gpu


def _run(monkeypatch, capsys, *args):
    monkeypatch.setattr(sys, "argv", ["bench.py", *args])
    bench.main()
    lines = [l for l in capsys.readouterr().out.strip().splitlines() if l.startswith("{")]
    assert len(lines) == 1, lines
    return json.loads(lines[0])


def _check_contract(d, steps, warmup, workload):
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["unit"] == "tokens/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["config"]["workload"] == workload
    tokens = d["config"]["batch"] * d["config"]["seqlen"]
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # value is tokens per second of the timed region: tokens / (ms per step)
    assert abs(d["value"] * d["ms_per_step"] * 1e-3 / tokens - 1) < 1e-6
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.HBM_PEAK_GBS
    assert 0 < r["frac"] < 1 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    # achieved = algorithmic bytes per launch / mean launch time
    assert abs(r["achieved"] - r["algorithmic_bytes_per_launch"] / (r["mean_launch_us"] * 1e-6) / 1e9) \
        < 0.01 * r["achieved"] + 1
    if d["plan"]["fused"]:   # the one-launch forward
        assert set(d["kernels"]) == {"forward_small"} and r["kernel"] == "forward_small"
    else:
        assert set(d["kernels"]) == {"chunk_cumsum", "state_pass", "group_scan", "chunk_out"}
    assert d["plan"]["sp_groups"] >= 1


def test_bench_line_small_bf16(monkeypatch, capsys):
    wl = "bf16_b2_L2048_H24_P64_N128_Q256"
    d = _run(monkeypatch, capsys, "--steps", "4", "--warmup", "2", "--kernel-reps", "8",
             "--cold-reps", "2", "--no-cpu-baseline", "--workload", wl)
    _check_contract(d, 4, 2, wl)
    assert d["dtype"] == "bf16" and d["plan_source"] == "cost model"
    assert d["cold"]["reps"] == 2 and d["cold"]["median_us"] > 0
    assert "cpu_baseline" not in d


def test_bench_line_fp32_with_cpu_baseline(monkeypatch, capsys):
    wl = "fp32_b1_L256_H4_P64_N64_Q64"
    d = _run(monkeypatch, capsys, "--steps", "3", "--warmup", "2", "--kernel-reps", "6",
             "--cold-reps", "0", "--cpu-budget", "0.5", "--workload", wl)
    _check_contract(d, 3, 2, wl)
    assert d["dtype"] == "f32" and d["plan"]["fused"] == 1
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s" and cb["value"] > 0
    assert cb["cores"] >= 1 and cb["threads"] >= 1 and cb["usable_cores"] >= 1 and cb["sample"]


def test_bench_line_autotuned(monkeypatch, capsys):
    wl = "bf16_b2_L2048_H24_P64_N128_Q256"
    d = _run(monkeypatch, capsys, "--steps", "4", "--warmup", "2", "--kernel-reps", "8",
             "--cold-reps", "0", "--no-cpu-baseline", "--autotune", "--workload", wl)
    _check_contract(d, 4, 2, wl)
    assert d["plan_source"] == "autotune"
    a = d["autotune"]
    assert a["candidates"] > 1 and a["forward_us"] <= a["default_forward_us"]
    assert d["plan"] in ssd.plan_candidates(ssd.make_problem(2, 2048, 24, 1, 64, 128, 256, "bf16"))


def test_bench_decode_step_line(monkeypatch, capsys):
    d = _run(monkeypatch, capsys, "--step", "4", "--steps", "5", "--warmup", "2", "--no-cpu-baseline")
    assert d["value"] > 0 and d["n_gpus"] == 1 and d["steps"] == 5
    assert 0 < d["roofline"]["frac"] < 1
