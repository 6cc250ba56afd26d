"""fp16 storage through the C ABI vs the fp64 oracle (needs an MI355X).

The kernels round the float64 rotation once to IEEE half precision.  Besides
the shapes of every tile mode, these tests aim at the values where rounding
first to fp32 and then to fp16 differs from one direct rounding (the kernels'
exact slow path), at fp16 subnormal results and at results past 65504 that
must become inf.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import packed_varlen_rotary_amd as P
import workloads as W
from tests.gpu_util import MIN_EXACT_FRACTION_AT_SCALE, bits16, check_against, check_every_element, f64

pytestmark = pytest.mark.gpu

DEV = "cuda"
LLAMA3 = dict(factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0, original_max_position=8192.0)


def cu_dev(cu):
    return torch.as_tensor(np.asarray(cu, dtype=np.int32), device=DEV)


def rotate(direction, q, k, cu, theta, **opts):
    (P.rope_qk_fwd if direction == 1 else P.rope_qk_bwd)(q, k, cu_dev(cu), theta, **opts)


def oracle_opts(opts):
    return dict(pos_offset=opts.get("pos_offset", 0), rotary_dim=opts.get("rotary_dim") or None,
                pairing="interleaved" if opts.get("interleaved") else "half", scaling=opts.get("llama3"))


def double_rounding_traps(ref):
    """Where rounding through fp32 (numpy's float64 -> float32 -> float16, each
    to nearest even) misses the oracle's single rounding to fp16."""
    direct = oracle.fp16_bits(oracle.fp16_rne(ref))
    via32 = ref.astype(np.float32).astype(np.float16).view(np.uint16)
    return direct != via32


def run_and_check(q, k, cu, theta, direction, **opts):
    xq, xk = f64(q), f64(k)
    rotate(direction, q, k, cu, theta, **opts)
    torch.cuda.synchronize()
    o = oracle_opts(opts)
    rq, rk = oracle.rope(xq, cu, theta, direction, **o), oracle.rope(xk, cu, theta, direction, **o)
    return (check_against(q, rq, f"q {opts}"), check_against(k, rk, f"k {opts}")), (rq, rk)


SHAPES = [
    # T, Hq, Hkv, D, tile mode
    (300, 6, 2, 16, "unit, half row of 1 chunk"),
    (513, 7, 1, 32, "unit, 2 chunks"),
    (400, 14, 2, 64, "unit, 4 chunks"),
    (301, 5, 1, 64, "unit, 4 chunks, 48 tasks per token: general addresses"),
    (150, 3, 2, 32, "unit, 2 chunks, 20 tasks per token: general addresses"),
    (257, 5, 3, 128, "pair tasks"),
    (129, 2, 2, 48, "pair tasks, 3 chunks"),
    (300, 5, 5, 80, "pair tasks, 5 chunks"),
    (64, 2, 2, 256, "pair tasks, 16 chunks"),
    (33, 4, 2, 512, "pair tasks, 32 chunks"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"T{s[0]}_H{s[1]}x{s[2]}_D{s[3]}")
@pytest.mark.parametrize("direction", [1, -1])
def test_fp16_shapes(shape, direction):
    T, Hq, Hkv, D, _ = shape
    q = W.randn((T, Hq, D), "fp16", seed=T * 7 + D, device=DEV)
    k = W.randn((T, Hkv, D), "fp16", seed=T * 11 + D, device=DEV)
    cu = [0, 1, T // 3, T // 3, T - 5]
    (sq, sk), _ = run_and_check(q, k, cu, 1e4, direction)
    assert sq["exact_fraction"] == 1.0 and sk["exact_fraction"] == 1.0, (sq, sk)


@pytest.mark.parametrize("D", [16, 64, 128, 80])
@pytest.mark.parametrize("direction", [1, -1])
def test_fp16_interleaved(D, direction):
    cu = [0, 1, 90, 90, 333, 500]
    q = W.randn((511, 7, D), "fp16", seed=50 + D, device=DEV)
    k = W.randn((511, 3, D), "fp16", seed=51 + D, device=DEV)
    (sq, sk), _ = run_and_check(q, k, cu, 1e4, direction, interleaved=True)
    assert sq["exact_fraction"] == 1.0 and sk["exact_fraction"] == 1.0, (sq, sk)


@pytest.mark.parametrize("D", [64, 128])
def test_fp16_double_rounding_traps_are_rounded_once(D):
    """About one value in 16,000 lands where fp32-then-fp16 rounding is wrong;
    a few million values give hundreds of them, every one must match."""
    T, Hq, Hkv = 4096, 16, 4
    q = W.randn((T, Hq, D), "fp16", seed=900 + D, device=DEV)
    k = W.randn((T, Hkv, D), "fp16", seed=901 + D, device=DEV)
    cu = [0, 1000, 2500, T]
    (sq, sk), (rq, rk) = run_and_check(q, k, cu, 1e6, 1)
    n_traps = 0
    for t, ref in ((q, rq), (k, rk)):
        traps = double_rounding_traps(ref)
        n_traps += int(traps.sum())
        want = oracle.fp16_bits(oracle.fp16_rne(ref))
        assert np.array_equal(bits16(t)[traps], want[traps])
    assert n_traps >= 50, n_traps
    assert sq["exact_fraction"] == 1.0 and sk["exact_fraction"] == 1.0, (sq, sk)


@pytest.mark.parametrize("D", [32, 128])
@pytest.mark.parametrize("direction", [1, -1])
def test_fp16_subnormal_results(D, direction):
    """Inputs near 2^-14: many results are fp16 subnormals (grid 2^-24)."""
    T, Hq, Hkv = 600, 6, 2
    q = W.randn((T, Hq, D), "fp16", seed=700 + D, device=DEV) * 2.0 ** -13
    k = W.randn((T, Hkv, D), "fp16", seed=701 + D, device=DEV) * 2.0 ** -13
    cu = [0, 250, T]
    (sq, sk), (rq, rk) = run_and_check(q, k, cu, 1e4, direction)
    sub = (np.abs(rq) < 2.0 ** -14) & (rq != 0)
    assert sub.mean() > 0.2, sub.mean()
    assert sq["exact_fraction"] == 1.0 and sk["exact_fraction"] == 1.0, (sq, sk)


@pytest.mark.parametrize("D", [64, 128])
def test_fp16_overflow_to_inf(D):
    """Inputs up to 65504: rotated results past the largest half become +-inf,
    those just below stay finite."""
    T, Hq, Hkv = 500, 4, 2
    q = (W.randn((T, Hq, D), "fp32", seed=800 + D, device=DEV) * 40000.0).clamp(-65504, 65504).half()
    k = (W.randn((T, Hkv, D), "fp32", seed=801 + D, device=DEV) * 40000.0).clamp(-65504, 65504).half()
    cu = [0, 100, T]
    (sq, sk), (rq, rk) = run_and_check(q, k, cu, 1e4, 1)
    assert np.isinf(oracle.fp16_rne(rq)).sum() > 0
    assert torch.isinf(q).sum().item() == int(np.isinf(oracle.fp16_rne(rq)).sum())
    assert not torch.isnan(q).any() and not torch.isnan(k).any()
    assert sq["exact_fraction"] == 1.0 and sk["exact_fraction"] == 1.0, (sq, sk)


@pytest.mark.parametrize("direction", [1, -1])
def test_fp16_all_options_together(direction):
    q = W.randn((720, 6, 128), "fp16", seed=81, device=DEV)
    k = W.randn((720, 2, 128), "fp16", seed=82, device=DEV)
    q0, k0 = q.clone(), k.clone()
    cu = [0, 100, 100, 620, 700]
    run_and_check(q, k, cu, 5e5, direction, pos_offset=4096, rotary_dim=64, interleaved=True, llama3=LLAMA3)
    assert torch.equal(q[:, :, 64:], q0[:, :, 64:]) and torch.equal(k[:, :, 64:], k0[:, :, 64:])


def test_fp16_partial_rotate_half():
    q = W.randn((300, 6, 128), "fp16", seed=83, device=DEV)
    k = W.randn((300, 2, 128), "fp16", seed=84, device=DEV)
    run_and_check(q, k, [0, 7, 150, 280], 1e4, 1, rotary_dim=32)


def test_fp16_shards_with_offset_equal_the_whole_sequence():
    T, Hq, Hkv, D, theta = 3000, 6, 2, 64, 1e6
    q = W.randn((T, Hq, D), "fp16", seed=5, device=DEV)
    k = W.randn((T, Hkv, D), "fp16", seed=6, device=DEV)
    qw, kw = q.clone(), k.clone()
    rotate(1, qw, kw, [0, T], theta)
    for a, b in ((0, 1111), (1111, 2048), (2048, T)):
        qs, ks = q[a:b].clone(), k[a:b].clone()
        rotate(1, qs, ks, [0, b - a], theta, pos_offset=a)
        assert torch.equal(qs, qw[a:b]) and torch.equal(ks, kw[a:b]), (a, b)


@pytest.mark.parametrize("direction", [1, -1])
def test_fp16_qwen3_8b_shape_every_element(direction):
    """Qwen3-8B-shaped packed batch (T = 65536, 32 + 8 heads, D = 128) stored in
    fp16, at full size in the benchmark's launch configuration; every element
    of q and k against the oracle, bit for bit."""
    w = dataclasses.replace(W.make_workload(3), dtype="fp16")
    names = ("q", "k") if direction == 1 else ("dq", "dk")
    t = W.make_tensors(w, names, device=DEV)
    before = {n: t[n].clone() for n in names}
    (P.rope_qk_fwd if direction == 1 else P.rope_qk_bwd)(t[names[0]], t[names[1]], cu_dev(w.cu_seqlens), w.theta)
    torch.cuda.synchronize()
    for n in names:
        s = check_every_element(before[n], t[n], w.cu_seqlens, w.theta, direction, f"fp16 {n}")
        print(n, s, flush=True)
        assert s["exact_fraction"] >= MIN_EXACT_FRACTION_AT_SCALE, s
    del t, before
    torch.cuda.empty_cache()
