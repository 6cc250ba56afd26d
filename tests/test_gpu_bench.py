"""The benchmark's JSON line on a GPU: one short run of bench.py (the
Qwen2.5-0.5B-shaped workload as the headline, no other workloads, no
stream ceiling, the fused norm on the same workload) prints one line with
every field of the contract, the roofline consistent with its own parts, a
parity check that passed, and the norm's timings consistent with their
bytes."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_prints_one_complete_json_line():
    import workloads as W

    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "2", "--table", "", "--no-ceiling",
           "--steps", "4", "--warmup", "2", "--cpu-seconds", "1", "--norm-table", "2"]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [ln for ln in out.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    w = W.make_workload(2)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 4 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == w.name
    # tokens/s of a step (forward and backward of one batch) against its wall time
    assert abs(d["value"] * d["ms_per_step"] / 1e3 - w.T) <= 1e-6 * w.T
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000
    assert 0 < r["achieved"] < r["peak"]
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-12
    assert r["traffic"] is None or r["traffic"] > 0
    # achieved = algorithmic bytes per launch / mean launch time
    k = d["kernel"]
    assert k["algorithmic_bytes_per_launch"] == w.bytes_per_pass
    assert abs(r["achieved"] - w.bytes_per_pass / (k["mean_launch_us"] * 1e-6) / 1e9) <= 1e-6 * r["achieved"]
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]
    p = d["parity"]
    assert p["ok"] is True and p["max_ulp"] <= 1 and p["tokens_checked"] == w.T
    # the fused norm: forward reads x and writes y, backward reads x and dy and writes dx
    (n,) = d["norm"]
    assert n["workload"] == w.name and n["calls_timed"] >= 20
    for name, nbytes in (("fwd", w.bytes_per_pass), ("bwd", 3 * w.bytes_per_pass // 2)):
        e = n[name]
        assert e["algorithmic_bytes"] == nbytes and e["us_per_call"] > 0
        assert abs(e["GB/s"] - nbytes / (e["us_per_call"] * 1e-6) / 1e9) <= 1e-6 * e["GB/s"]
        assert abs(e["frac"] - e["GB/s"] / 8000) < 1e-12 and 0 < e["frac"] < 1


@pytest.mark.gpu
def test_bench_without_the_oracle_leg_reports_no_parity():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "2", "--table", "", "--no-ceiling",
           "--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--norm-table", ""]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    d = json.loads(out.stdout.strip().splitlines()[-1])
    assert d["cpu_baseline"] is None and "skipped" in d["parity"] and d["norm"] == []
