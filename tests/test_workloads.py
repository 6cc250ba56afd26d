"""Seeded input generators: well-formed metadata, exact sizes, reproducibility, valid packing."""

import numpy as np
import pytest
import torch

import workloads as W


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_cu_seqlens_well_formed(cfg):
    w = W.make_workload(cfg)
    cu = w.cu_seqlens
    assert cu.dtype == np.int32
    assert cu[0] == 0 and cu[-1] == w.T
    assert np.all(np.diff(cu.astype(np.int64)) > 0)
    assert w.D % 2 == 0
    assert w.bytes_per_pass == 2 * (w.Hq + w.Hkv) * w.D * w.elem_size * w.T


def test_shapes_match_the_named_models():
    expect = {1: (256, 14, 2, 64, 1e6, "fp32"), 2: (16384, 14, 2, 64, 1e6, "bf16"),
              3: (65536, 32, 8, 128, 1e6, "bf16"), 4: (131072, 64, 8, 128, 1e6, "bf16"),
              5: (524288, 32, 8, 128, 5e5, "bf16")}
    for cfg, (T, Hq, Hkv, D, theta, dt) in expect.items():
        w = W.make_workload(cfg)
        assert (w.T, w.Hq, w.Hkv, w.D, w.theta, w.dtype) == (T, Hq, Hkv, D, theta, dt)
    assert list(W.make_workload(1).cu_seqlens) == [0, 7, 40, 104, 256]
    assert W.make_workload(5).T * 32 * 128 == 2 ** 31


def test_reproducible():
    for cfg in (2, 3, 4):
        assert np.array_equal(W.make_workload(cfg).cu_seqlens, W.make_workload(cfg).cu_seqlens)
    w = W.make_workload(1)
    a = W.make_tensors(w, ("q", "k"))
    b = W.make_tensors(w, ("q", "k"))
    assert torch.equal(a["q"], b["q"]) and torch.equal(a["k"], b["k"])
    assert not torch.equal(a["q"][:, :2], a["k"])


def test_length_distributions():
    L3 = np.diff(W.make_workload(3).cu_seqlens)
    assert L3[:-1].min() >= 16 and L3.max() <= 4096
    assert 150 < np.median(L3) < 420  # log-normal with median 256
    L4 = np.diff(W.make_workload(4).cu_seqlens)[:-1]
    assert np.all(((L4 >= 64) & (L4 <= 1024)) | ((L4 >= 4096) & (L4 <= 16384)))


def test_best_fit_decreasing_is_valid():
    rng = np.random.default_rng(3)
    lengths = rng.integers(1, 100, size=300)
    cap = 256
    bins = W.best_fit_decreasing(lengths, cap)
    placed = sorted(i for b in bins for i in b)
    assert placed == list(range(len(lengths)))
    for b in bins:
        assert sum(int(lengths[i]) for i in b) <= cap
    # no two bins could be merged (a property any best-fit packing has)
    fills = sorted(sum(int(lengths[i]) for i in b) for b in bins)
    assert fills[0] + fills[1] > cap


def test_best_fit_decreasing_textbook_case():
    # decreasing order 7,6,5,4,3,2 into capacity 10: 7->A, 6->B, 5->C, 4->B (room 4 = best), 3->A, 2->C
    bins = W.best_fit_decreasing([5, 7, 3, 6, 2, 4], 10)
    assert [[ [5, 7, 3, 6, 2, 4][i] for i in b] for b in bins] == [[7, 3], [6, 4], [5, 2]]


def test_qwen_rows():
    graded, rows = W.qwen25_05b_rows()
    for r in rows:
        assert sum(r) == 16384
    assert len(rows[graded]) == max(len(r) for r in rows)
    for i in range(len(rows)):
        w = W.make_workload(2, row=i)
        assert w.cu_seqlens[-1] == 16384
