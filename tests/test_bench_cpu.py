"""The benchmark's host-only legs: the oracle timing (the cpu_baseline of the
JSON line, and the per-workload table of --cpu-table) runs the oracle on the
workload's own seeded inputs and reports what it timed."""

import json
import os
import subprocess
import sys

import numpy as np

import bench
import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_inputs_are_the_workloads_chunks():
    w = W.make_workload(2)
    chunks = bench.oracle_inputs(w, 3, 1024)
    assert len(chunks) == 3
    pos_all = oracle.segment_positions(w.cu_seqlens, w.T)
    for i, (pos, xs) in enumerate(chunks):
        assert np.array_equal(pos, pos_all[i * 1024:(i + 1) * 1024])
        assert [x.shape for x in xs] == [(1024, w.Hq, w.D), (1024, w.Hkv, w.D)]
        for x in xs:  # bf16 values: rounding again changes nothing
            assert np.array_equal(oracle.bf16_rne(x), x)


def test_oracle_pass_counts_each_chunks_tokens_once():
    w = W.make_workload(1)
    (pos, xs), = bench.oracle_inputs(w, 4, 1024)  # 256 tokens: one chunk
    assert len(pos) == w.T
    assert bench.oracle_pass(w, pos, xs, (1, -1)) == w.T
    tokens, dt = bench.oracle_rate(w, [(pos, xs)], (1,), 1, 0.05)
    assert tokens % w.T == 0 and tokens >= w.T and dt >= 0.05


def test_cpu_table_prints_one_line_per_workload():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--cpu-table", "--table", "1,2",
                          "--cpu-seconds", "0.2"], capture_output=True, text=True, check=True, timeout=300)
    rows = [json.loads(line) for line in out.stdout.splitlines() if line.strip()]
    assert [r["workload"] for r in rows] == [W.make_workload(c).name for c in (1, 2)]
    for r in rows:
        assert r["threads"] >= 1 and r["host_cores"] >= r["threads"]
        for d in ("fwd", "bwd"):
            assert r[d]["pool_tokens"] > 0 and r[d]["pool_tokens_per_s"] > 0 and r[d]["single_tokens_per_s"] > 0


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=300)
    assert out.returncode == 2
    assert out.stdout == ""
    assert "one GPU" in out.stderr


def _oracle_sample(w, idx):
    """A parity sample as the GPU run would hand it over, with the oracle's
    own outputs in place of the GPU's (inputs: the workload's seeded q, k and
    fresh gradients at the sampled tokens)."""
    rng = np.random.default_rng(5)
    pos = oracle.segment_positions(w.cu_seqlens, w.T)[idx]
    x, out = {}, {}
    for n, h, d in (("q", w.Hq, 1), ("k", w.Hkv, 1), ("dq", w.Hq, -1), ("dk", w.Hkv, -1)):
        xi = oracle.bf16_rne(rng.standard_normal((len(idx), h, w.D)))
        x[n] = xi
        out[n] = oracle.bf16_bits(oracle.bf16_rne(oracle.rotate(xi, pos, w.theta, d)))
    return {"idx": idx, "x": x, "out": out}


def test_oracle_parity_counts_and_bounds_ulp_differences():
    w = W.make_workload(2)
    idx = np.array([0, 1, 7, 500, w.T - 1])
    s = _oracle_sample(w, idx)
    p = bench.oracle_parity(w, s)
    assert p == {"max_ulp": 0, "max_abs": 0.0, "exact_fraction": 1.0, "tokens_checked": 5, "ok": True}
    # one element one bf16 ulp off (next bit pattern away from zero): still within
    # the bound, and counted as not bit-exact
    s["out"]["k"][2, 1, 3] += 1
    p = bench.oracle_parity(w, s)
    n = sum(o.size for o in s["out"].values())
    assert p["max_ulp"] == 1 and p["ok"] is True and abs(p["exact_fraction"] - (n - 1) / n) < 1e-15
    # two ulp off: the check fails
    s["out"]["dq"][4, 0, 0] += 2
    p = bench.oracle_parity(w, s)
    assert p["max_ulp"] == 2 and p["ok"] is False
