"""The benchmark's JSON line on the GPU: one short in-process run of bench.py's main()."""

import json
import sys

import pytest
import torch

from tests.parity import say

pytestmark = pytest.mark.gpu

KEYS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
        "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline")


def test_bench_line_contract(capsys, monkeypatch):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench

    say("[gpu] bench.py main, batch8, 3 steps")
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "batch8", "--steps", "3", "--warmup", "1",
                                      "--no-flush", "--settle-ms", "50", "--cpu-budget", "0.5"])
    assert bench.main() == 0
    out = capsys.readouterr().out.strip().splitlines()
    r = json.loads(out[-1])
    for key in KEYS:
        assert key in r, key
    assert r["n_gpus"] == 1 and r["steps"] == 3 and r["warmup"] == 1
    assert r["config"]["workload"].startswith("batch8") and r["dtype"] == "bf16"
    assert r["value"] > 0 and r["ms_per_step"] > 0 and r["higher_is_better"] is True
    ro = r["roofline"]
    assert ro["bound"] == "hbm" and ro["unit"] == "GB/s" and ro["peak"] == 8000.0
    assert 0 < ro["frac"] < 1 and abs(ro["frac"] - ro["achieved"] / ro["peak"]) < 1e-3
    # frac counts the effective bytes Q + K + V + O + LSE once, never the partials.
    assert ro["algorithmic_bytes_per_launch"] == r["effective_bytes"]
    assert abs(ro["achieved"] - r["effective_bytes"] / (ro["ms_per_launch"] * 1e-3) / 1e9) < 0.02 * ro["achieved"]
    assert ro["partial_workspace_bytes_uncredited"] > 0
    assert r["cold_cache"] is False and "sub_runs" not in r
    cb = r["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert cb["complete"] == (cb["groups_timed"] == cb["groups_total"] == 64) and cb["cpu_model"]
    ex = r["lpt"]["executed"]
    assert ex["static_lists_page_cost"] == round(r["lpt"]["imbalance"], 6)
    # The backward call is timed by default (bf16 workload), with fp32 and bf16 dK/dV.
    bw = r["backward"]
    for key in ("fp32_dkv", "bf16_dkv"):
        assert bw[key]["ms_per_call"] > 0 and 0 < bw[key]["roofline_fraction"] < 1
    assert bw["bf16_dkv"]["bytes"] < bw["fp32_dkv"]["bytes"]
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_bench_line_cold_cache_and_sub_runs(capsys, monkeypatch):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench

    say("[gpu] bench.py main, batch8 with a sub-run, flushed steps")
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "batch8", "--sub-runs", "small", "--steps", "2",
                                      "--warmup", "1", "--settle-ms", "20", "--no-cpu-baseline"])
    assert bench.main() == 0
    r = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert r["cold_cache"] is True and r["ms_per_step_min"] <= r["ms_per_step_median"]
    sub = r["sub_runs"]["small"]
    assert sub["workload"].startswith("small") and sub["ms_per_step"] > 0 and sub["roofline"]["frac"] > 0
    assert "cpu_baseline" not in r
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
