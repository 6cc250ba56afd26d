"""Variants through the C ABI vs the fp64 oracle (needs an MI355X): position
offset of a token shard, partial rotary dim, interleaved pairing, the
Llama 3.1 frequency rescaling and float32-convention angles, each alone and
combined, forward and backward.
"""

import numpy as np
import pytest
import torch

import oracle
import packed_varlen_rotary_amd as P
import workloads as W
from tests.gpu_util import check_against, f64

pytestmark = pytest.mark.gpu

DEV = "cuda"
LLAMA3 = dict(factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0, original_max_position=8192.0)


def cu_dev(cu):
    return torch.as_tensor(np.asarray(cu, dtype=np.int32), device=DEV)


def rotate(direction, q, k, cu, theta, **opts):
    (P.rope_qk_fwd if direction == 1 else P.rope_qk_bwd)(q, k, cu_dev(cu), theta, **opts)


def oracle_opts(opts):
    """rope_qk_fwd keyword options -> oracle.rope keyword options."""
    return dict(pos_offset=opts.get("pos_offset", 0), rotary_dim=opts.get("rotary_dim") or None,
                pairing="interleaved" if opts.get("interleaved") else "half", scaling=opts.get("llama3"),
                freq_precision="fp32" if opts.get("freq_fp32") else "fp64")


def check_case(T, Hq, Hkv, D, dt, cu, theta, direction, seed, **opts):
    q = W.randn((T, Hq, D), dt, seed=seed, device=DEV)
    k = W.randn((T, Hkv, D), dt, seed=seed + 1, device=DEV)
    return check_case_tensors(q, k, cu, theta, direction, **opts)


def check_case_tensors(q, k, cu, theta, direction, **opts):
    xq, xk = f64(q), f64(k)
    rotate(direction, q, k, cu, theta, **opts)
    torch.cuda.synchronize()
    o = oracle_opts(opts)
    sq = check_against(q, oracle.rope(xq, cu, theta, direction, **o), f"q {opts}")
    sk = check_against(k, oracle.rope(xk, cu, theta, direction, **o), f"k {opts}")
    return sq, sk


# ---------------------------------------------------------------------------
# position offset (token shards)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("D,dt,interleaved", [(64, "bf16", False), (128, "bf16", False), (64, "fp32", False),
                                              (128, "bf16", True), (32, "fp32", True)])
def test_shards_with_offset_equal_the_whole_sequence(D, dt, interleaved):
    """One 3,000-token sequence rotated whole, and as three token shards whose
    later shards pass pos_offset = their global start: bit-identical."""
    T, Hq, Hkv, theta = 3000, 6, 2, 1e6
    q = W.randn((T, Hq, D), dt, seed=D, device=DEV)
    k = W.randn((T, Hkv, D), dt, seed=D + 1, device=DEV)
    qw, kw = q.clone(), k.clone()
    rotate(1, qw, kw, [0, T], theta, interleaved=interleaved)
    for a, b in ((0, 1111), (1111, 2048), (2048, T)):
        qs, ks = q[a:b].clone(), k[a:b].clone()
        rotate(1, qs, ks, [0, b - a], theta, pos_offset=a, interleaved=interleaved)
        assert torch.equal(qs, qw[a:b]) and torch.equal(ks, kw[a:b]), (a, b)


@pytest.mark.parametrize("direction", [1, -1])
def test_offset_moves_segment_zero_only(direction):
    cu = [3, 40, 40, 170, 400, 405]
    s = check_case(420, 5, 3, 64, "bf16", cu, 1e6, direction, 31, pos_offset=123456)
    assert s[0]["exact_fraction"] == 1.0 and s[1]["exact_fraction"] == 1.0


def test_offset_near_the_position_limit():
    T = 64
    check_case(T, 2, 1, 128, "bf16", [0, T], 5e5, 1, 37, pos_offset=2 ** 31 - 1 - T)


# ---------------------------------------------------------------------------
# partial rotary dim
# ---------------------------------------------------------------------------

PARTIAL = [
    # T, Hq, Hkv, D, r, dtype, interleaved
    (300, 6, 2, 128, 64, "bf16", False),  # rotated half row of 4 chunks: chunk tasks on part of a row
    (300, 6, 2, 128, 32, "bf16", False),  # 2 chunks
    (257, 5, 3, 256, 96, "bf16", False),  # 6 chunks: chunk-pair tasks
    (200, 4, 4, 80, 48, "fp32", False),
    (257, 7, 1, 96, 32, "bf16", True),
    (190, 3, 2, 64, 16, "fp32", True),
]


@pytest.mark.parametrize("case", PARTIAL, ids=lambda c: f"D{c[3]}_r{c[4]}_{c[5]}_{'il' if c[6] else 'half'}")
@pytest.mark.parametrize("direction", [1, -1])
def test_partial_rotary_dim(case, direction):
    T, Hq, Hkv, D, r, dt, il = case
    cu = [0, 7, 150, T - 20]
    q = W.randn((T, Hq, D), dt, seed=r, device=DEV)
    k = W.randn((T, Hkv, D), dt, seed=r + 1, device=DEV)
    q0, k0 = q.clone(), k.clone()
    xq, xk = f64(q), f64(k)
    rotate(direction, q, k, cu, 1e4, rotary_dim=r, interleaved=il)
    torch.cuda.synchronize()
    assert torch.equal(q[:, :, r:], q0[:, :, r:]) and torch.equal(k[:, :, r:], k0[:, :, r:])  # tail untouched
    o = oracle_opts(dict(rotary_dim=r, interleaved=il))
    check_against(q, oracle.rope(xq, cu, 1e4, direction, **o), "q")
    check_against(k, oracle.rope(xk, cu, 1e4, direction, **o), "k")


LARGE_CHUNK_TASKS = [
    # T, Hq, Hkv, D, dtype, options: chunk-task launches of more than 2^21
    # tasks (2^20 for rows rotating under a line of a longer head), which
    # take fewer chunks per lane than smaller ones
    (20000, 14, 2, 64, "bf16", {}),                     # 4 chunks per lane
    (20000, 14, 2, 64, "fp16", {}),
    (40000, 12, 4, 32, "bf16", {}),                     # half rows of 2 chunks, 4 per lane
    (20000, 14, 2, 64, "bf16", {"interleaved": True}),  # interleaved rows of 8 chunks, 4 per lane
    (20000, 14, 2, 64, "bf16", {"rotary_dim": 32}),     # rotated rows of half a line: 1 chunk per lane
    (20000, 14, 2, 64, "fp16", {"rotary_dim": 32}),
    (20000, 28, 4, 32, "bf16", {"rotary_dim": 16}),     # half rows of 1 chunk, 1 per lane
    (20000, 14, 2, 128, "bf16", {"rotary_dim": 64}),    # a whole line of a longer head: 4 per lane
    (16384, 14, 2, 64, "bf16", {}),                     # exactly 2^21 tasks: still 8 per lane
    (16385, 14, 2, 64, "bf16", {}),                     # one token more: 4 per lane
    (16384, 14, 2, 64, "bf16", {"rotary_dim": 32}),     # exactly 2^20 tasks of part rows: 8 per lane
    (16385, 14, 2, 64, "bf16", {"rotary_dim": 32}),     # one token more: 1 per lane
]


@pytest.mark.parametrize("case", LARGE_CHUNK_TASKS,
                         ids=lambda c: f"T{c[0]}_H{c[1]}x{c[2]}_D{c[3]}_{c[4]}" + "".join(f"_{o}" for o in c[5]))
@pytest.mark.parametrize("direction", [1, -1])
def test_large_chunk_task_launches(case, direction):
    """Every element of launches large enough for the lane counts of large
    chunk-task launches, against the oracle: ragged segments, tokens outside
    at both ends, a ragged last tile; partial rotary dims leave the tail alone."""
    T, Hq, Hkv, D, dt, opts = case
    rng = np.random.default_rng(T + Hq + D)
    lengths = rng.integers(1, 3000, size=T // 500)
    cu = np.concatenate([[0], np.cumsum(lengths)]) + 5
    cu = cu[cu <= T - 3]
    q = W.randn((T, Hq, D), dt, seed=T + 1, device=DEV)
    k = W.randn((T, Hkv, D), dt, seed=T + 2, device=DEV)
    q0, k0 = q.clone(), k.clone()
    sq, sk = check_case_tensors(q, k, cu, 5e5, direction, **opts)
    if dt == "bf16":
        assert sq["exact_fraction"] == 1.0 and sk["exact_fraction"] == 1.0
    r = opts.get("rotary_dim")
    if r:
        assert torch.equal(q[:, :, r:], q0[:, :, r:]) and torch.equal(k[:, :, r:], k0[:, :, r:])


# ---------------------------------------------------------------------------
# interleaved pairing
# ---------------------------------------------------------------------------

INTERLEAVED = [(16, "bf16"), (32, "bf16"), (64, "bf16"), (128, "bf16"), (80, "bf16"), (256, "bf16"),
               (8, "fp32"), (64, "fp32"), (72, "fp32"), (128, "fp32")]


@pytest.mark.parametrize("D,dt", INTERLEAVED)
@pytest.mark.parametrize("direction", [1, -1])
def test_interleaved_pairing(D, dt, direction):
    cu = [0, 1, 90, 90, 333, 500]
    s = check_case(511, 7, 3, D, dt, cu, 1e4, direction, 50 + D, interleaved=True)
    if dt == "bf16":
        assert s[0]["exact_fraction"] == 1.0 and s[1]["exact_fraction"] == 1.0


def test_interleaved_is_rotate_half_on_a_permuted_head():
    """Interleaved RoPE of x equals rotate_half RoPE of x with each head reordered
    (2i -> i, 2i+1 -> i + D/2), then put back: same angles, same operations."""
    T, H, D = 400, 8, 64
    x = W.randn((T, H, D), "bf16", seed=3, device=DEV)
    perm = torch.cat([torch.arange(0, D, 2), torch.arange(1, D, 2)]).to(DEV)
    a = x.clone()
    k0 = torch.empty((T, 0, D), dtype=x.dtype, device=DEV)
    P.rope_qk_fwd(a, k0, cu_dev([0, 150, T]), 1e6, interleaved=True)
    b = x[:, :, perm].contiguous()
    P.rope_qk_fwd(b, k0, cu_dev([0, 150, T]), 1e6)
    inv = torch.argsort(perm)
    assert torch.equal(a, b[:, :, inv])


# ---------------------------------------------------------------------------
# Llama 3.1 frequency rescaling, and everything together
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("direction", [1, -1])
def test_llama3_scaling_long_positions(direction):
    """Llama-3.1-8B-shaped heads at positions around 200K (an offset shard)."""
    s = check_case(1500, 32, 8, 128, "bf16", [0, 1500], 5e5, direction, 71, pos_offset=200_000, llama3=LLAMA3)
    assert s[0]["exact_fraction"] > 0.9999 and s[1]["exact_fraction"] > 0.9999


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("direction", [1, -1])
def test_all_options_together(dt, direction):
    cu = [0, 100, 100, 620, 700]
    check_case(720, 6, 2, 128, dt, cu, 5e5, direction, 81, pos_offset=4096, rotary_dim=64, interleaved=True,
               llama3=LLAMA3)


def test_options_struct_entry_points():
    """The _opt entry points with an explicit struct, and with NULL (= the plain call)."""
    T, Hq, Hkv, D = 256, 4, 2, 64
    q = W.randn((T, Hq, D), "bf16", seed=90, device=DEV)
    k = W.randn((T, Hkv, D), "bf16", seed=91, device=DEV)
    cu = cu_dev([0, 100, T])
    a, b = (q.clone(), k.clone()), (q.clone(), k.clone())
    P.rope_qk_fwd_opt(a[0], a[1], cu, 1e6, None)
    P.rope_qk_fwd(b[0], b[1], cu, 1e6)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    c = (q.clone(), k.clone())
    P.rope_qk_fwd_opt(c[0], c[1], cu, 1e6, P.make_options(pos_offset=7, rotary_dim=32))
    torch.cuda.synchronize()
    o = oracle_opts(dict(pos_offset=7, rotary_dim=32))
    check_against(c[0], oracle.rope(f64(q), [0, 100, T], 1e6, 1, **o), "q")
    check_against(c[1], oracle.rope(f64(k), [0, 100, T], 1e6, 1, **o), "k")


def test_backward_undoes_forward_with_options():
    T, Hq, Hkv, D = 600, 4, 2, 128
    q = W.randn((T, Hq, D), "fp32", seed=95, device=DEV)
    k = W.randn((T, Hkv, D), "fp32", seed=96, device=DEV)
    q0, k0 = q.clone(), k.clone()
    opts = dict(pos_offset=1000, rotary_dim=96, interleaved=True, llama3=LLAMA3)
    cu = cu_dev([0, 250, T])
    P.rope_qk_fwd(q, k, cu, 5e5, **opts)
    P.rope_qk_bwd(q, k, cu, 5e5, **opts)
    torch.cuda.synchronize()
    assert float((q - q0).abs().max()) <= 1e-6 and float((k - k0).abs().max()) <= 1e-6


# ---------------------------------------------------------------------------
# float32-convention angles
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["bf16", "fp32", "fp16"])
@pytest.mark.parametrize("direction", [1, -1])
def test_fp32_angles_long_positions(dt, direction):
    """Positions around 5e5 (an offset shard of a long sequence), where the
    float32 angles differ from the float64 ones by up to ~0.03 rad."""
    T, Hq, Hkv, D = 700, 8, 2, 128
    q = W.randn((T, Hq, D), dt, seed=61, device=DEV)
    k = W.randn((T, Hkv, D), dt, seed=62, device=DEV)
    q64, k64 = q.clone(), k.clone()
    s = check_case_tensors(q, k, [0, 300, T], 5e5, direction, pos_offset=500_000, freq_fp32=True)
    if dt != "fp32":
        assert s[0]["exact_fraction"] == 1.0 and s[1]["exact_fraction"] == 1.0, s
    rotate(direction, q64, k64, [0, 300, T], 5e5, pos_offset=500_000)
    assert not torch.equal(q, q64)  # the two conventions really differ here


def test_fp32_angles_across_2_pow_24():
    """Positions 2^24 - 150 .. 2^24 + 150: past 2^24 the float32 position itself rounds."""
    T = 300
    s = check_case(T, 4, 2, 64, "bf16", [0, T], 1e6, 1, 63, pos_offset=2 ** 24 - 150, freq_fp32=True)
    assert s[0]["exact_fraction"] == 1.0 and s[1]["exact_fraction"] == 1.0, s


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_fp32_angles_with_every_option(dt):
    cu = [0, 100, 100, 620, 700]
    check_case(720, 6, 2, 128, dt, cu, 5e5, 1, 64, pos_offset=40960, rotary_dim=64, interleaved=True,
               llama3=LLAMA3, freq_fp32=True)


def test_fp32_angles_equal_fp64_where_exact():
    """Base 2^16 at D = 4: frequencies 1 and 2^-8 and every product below 2^24
    are exact in float32, so both conventions give identical results."""
    T = 512
    q = W.randn((T, 3, 4 * 8), "fp32", seed=65, device=DEV)[:, :, :4].contiguous()
    k = torch.empty((T, 0, 4), dtype=q.dtype, device=DEV)
    a, b = q.clone(), q.clone()
    # D = 4 fp32 has 8-byte half rows: rotate_half needs 16; interleaved pairs need r * 4 = 16 bytes
    rotate(1, a, k, [0, T], 2.0 ** 16, interleaved=True, freq_fp32=True, pos_offset=2 ** 24 - T)
    rotate(1, b, k, [0, T], 2.0 ** 16, interleaved=True, pos_offset=2 ** 24 - T)
    assert torch.equal(a, b)
