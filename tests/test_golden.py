"""Regression lock: the oracle still reproduces the stored tiny fixture bit for bit."""

import json
import os

import numpy as np

import oracle

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_tiny_fixture():
    with open(os.path.join(HERE, "tiny_rope_oracle.json")) as f:
        g = json.load(f)
    x = np.array(g["x"], dtype=np.float64)
    cu = np.array(g["cu_seqlens"])
    assert list(oracle.segment_positions(cu, g["T"])) == g["positions"]
    for name, d in (("fwd", 1), ("bwd", -1)):
        y = oracle.rope(x, cu, g["theta"], d).ravel()
        assert [float.hex(float(v)) for v in y] == g[name]
        assert [int(b) for b in oracle.bf16_bits(oracle.bf16_rne(y))] == g[name + "_bf16_bits"]
    # token 5 lies outside every sequence and the first token of each sequence is at position 0
    assert np.array_equal(np.array([float.fromhex(v) for v in g["fwd"]]).reshape(x.shape)[[0, 3, 5]], x[[0, 3, 5]])
