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
