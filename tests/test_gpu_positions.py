"""Positions through the kernels' own code (needs an MI355X).

The rotation kernels find each tile's first sequence with a binary search
of cu_seqlens and then scan the sequence starts inside the tile; the norm
forward does the same per tile, and the norm backward carries a cursor into
cu_seqlens from tile to tile along each workgroup's run.  The test hooks
(rope_qk_tile_positions, rope_qk_norm_tile_positions) run exactly that code,
in the tile decomposition of a given call, and report every tile's first
token and the positions of the tokens it touches.  Every position is
compared with the oracle's segment positions bit for bit, the tiles must be
in token order and cover every token, and tokens in no sequence must read -1
(the auto-packing paragraph of the Unsloth article: length metadata keeps
packed samples apart).
"""

import numpy as np
import pytest
import torch

import oracle
import packed_varlen_rotary_amd as P
import workloads as W
from tests import oracle_pins

pytestmark = pytest.mark.gpu

DEV = "cuda"


def metadata_cases():
    cases = [(np.asarray(cu), T) for cu, T in oracle_pins.POSITION_CASES]
    for cfg in (1, 2, 3, 4, 5):
        w = W.make_workload(cfg)
        cases.append((w.cu_seqlens, w.T))
    rng = np.random.default_rng(7)
    many = np.sort(rng.integers(0, 5000, size=3000))  # thousands of segments, many of them empty
    cases.append((np.concatenate([[0], many, [5000]]), 5003))
    short = np.cumsum(rng.integers(0, 8, size=2500))  # sequences of 0-7 tokens: several starts in every tile
    cases.append((np.concatenate([[3], 3 + short]), int(3 + short[-1] + 11)))  # tokens outside at both ends
    return [(np.asarray(cu, dtype=np.int32), int(T)) for cu, T in cases]


def check_rows(rows, cu, T, pos_offset, what):
    """Each hook row against the oracle; rows in token order, covering every token."""
    rows = rows.cpu().numpy().astype(np.int64)
    want = oracle.segment_positions(cu, T, pos_offset)
    t0 = rows[:, 0]
    vals = rows[:, 1:]
    written = vals != P.TILE_ROW_UNWRITTEN
    n = written.sum(axis=1)
    cols = np.arange(vals.shape[1])
    assert np.array_equal(written, cols[None, :] < n[:, None]), f"{what}: rows are not written as a prefix"
    assert (n >= 1).all() and (t0 >= 0).all() and (t0 + n <= T).all(), what
    assert (np.diff(t0) >= 0).all(), f"{what}: tiles out of token order"
    tok = t0[:, None] + cols[None, :]
    got = vals[written]
    ref = want[np.minimum(tok, T - 1)][written]
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{what}: {bad.size} positions differ (first at token {tok[written][bad[0]]})"
    covered = np.zeros(T + 1, dtype=np.int64)
    np.add.at(covered, t0, 1)
    np.add.at(covered, t0 + n, -1)
    assert (np.cumsum(covered)[:T] >= 1).all(), f"{what}: a token no tile touches"
    return rows.shape[0]


ROTATION_SHAPES = [
    # Hq, Hkv, D, dtype code, options (keyword arguments of make_options)
    (14, 2, 64, P.ROPE_QK_BF16, {}),              # unit tiles (the Qwen2.5-0.5B shape): 8 chunks per lane, 4 past 2^21 tasks
    (14, 2, 64, P.ROPE_QK_BF16, {"rotary_dim": 32}),  # rotated rows of half a line: 1 chunk per lane past 2^20 tasks
    (32, 8, 128, P.ROPE_QK_BF16, {}),             # pair tiles, tiles starting inside tokens (Qwen3-8B)
    (64, 8, 128, P.ROPE_QK_BF16, {}),             # pair tiles, 576 tasks per token (Qwen3-32B)
    (144, 16, 128, P.ROPE_QK_BF16, {}),           # a token spans several tiles
    (7, 3, 96, P.ROPE_QK_BF16, {}),               # chunk pairs, 6 chunks per half row
    (3, 1, 16, P.ROPE_QK_FP32, {}),               # fp32 unit tiles
    (5, 5, 80, P.ROPE_QK_FP16, {}),
    (14, 2, 64, P.ROPE_QK_BF16, {"interleaved": True}),
    (14, 2, 128, P.ROPE_QK_BF16, {"rotary_dim": 64}),
    (2, 2, 512, P.ROPE_QK_BF16, {}),              # 16 tokens per tile at most (the table's limit)
]


@pytest.mark.parametrize("shape", ROTATION_SHAPES, ids=lambda s: f"H{s[0]}x{s[1]}_D{s[2]}_dt{s[3]}_{s[4]}")
def test_rotation_tile_positions(shape):
    Hq, Hkv, D, dt, opts = shape
    for cu, T in metadata_cases():
        cu_d = torch.as_tensor(cu, device=DEV)
        for pos_offset in (0, 1, 100003):
            if pos_offset + T > 2 ** 31 - 1:
                continue
            o = P.make_options(pos_offset=pos_offset, **opts)
            rows = P.rope_qk_tile_positions(cu_d, T, Hq, Hkv, D, dt, o)
            if cu.size == 1:  # no sequence: the call launches nothing
                assert rows.numel() == 0
                continue
            check_rows(rows, cu, T, pos_offset, f"rotation {shape} T={T} nseq={cu.size - 1} offset={pos_offset}")


LANE_COUNTS = [
    # T, Hq, Hkv, D, dtype code, options, tasks per token, chunks per lane
    (16384, 14, 2, 64, P.ROPE_QK_BF16, {}, 128, 8),                     # 2^21 tasks: small
    (16385, 14, 2, 64, P.ROPE_QK_BF16, {}, 128, 4),
    (16384, 14, 2, 64, P.ROPE_QK_BF16, {"rotary_dim": 32}, 64, 8),      # 2^20 tasks of part rows: small
    (16385, 14, 2, 64, P.ROPE_QK_BF16, {"rotary_dim": 32}, 64, 1),
    (16385, 14, 2, 64, P.ROPE_QK_FP16, {"rotary_dim": 32}, 64, 1),
    (16384, 14, 2, 64, P.ROPE_QK_BF16, {"interleaved": True}, 128, 8),
    (16385, 14, 2, 64, P.ROPE_QK_BF16, {"interleaved": True}, 128, 4),
    (20000, 14, 2, 128, P.ROPE_QK_BF16, {"rotary_dim": 64}, 128, 4),    # one whole line of a longer head
    (20000, 14, 2, 32, P.ROPE_QK_FP32, {}, 128, 4),                     # fp32 chunk tiles: 4 at any size
]


@pytest.mark.parametrize("case", LANE_COUNTS,
                         ids=lambda c: f"T{c[0]}_D{c[3]}_dt{c[4]}" + "".join(f"_{k}{v}" for k, v in c[5].items()))
def test_chunk_task_lane_counts(case):
    """The tile decomposition of chunk-task calls, as the hook runs it: 256
    lanes times the chunks per lane that the launch's size and row shape
    select (8 up to 2^21 tasks, 2^20 for rows rotating under a line of a
    longer head; 4, or 1 for those rows, beyond)."""
    T, Hq, Hkv, D, dt, opts, tpt, lanes = case
    cu = torch.as_tensor(np.array([0, T], dtype=np.int32), device=DEV)
    rows = P.rope_qk_tile_positions(cu, T, Hq, Hkv, D, dt, P.make_options(**opts))
    assert rows.shape[0] == -(-T * tpt // (256 * lanes)), (case, rows.shape)
    check_rows(rows, np.array([0, T], dtype=np.int32), T, 0, f"lane counts {case}")


NORM_SHAPES = [
    (32, 8, 128, P.ROPE_QK_BF16),
    (14, 2, 64, P.ROPE_QK_BF16),
    (6, 2, 128, P.ROPE_QK_FP32),
    (3, 2, 512, P.ROPE_QK_BF16),
    (7, 1, 16, P.ROPE_QK_FP16),
]


@pytest.mark.parametrize("backward", [False, True], ids=["fwd", "bwd"])
@pytest.mark.parametrize("shape", NORM_SHAPES, ids=lambda s: f"H{s[0]}x{s[1]}_D{s[2]}_dt{s[3]}")
def test_norm_tile_positions(shape, backward):
    """The norm forward's per-tile search and the norm backward's cursor
    (carried along each workgroup's run of tiles, across q's tiles into k's)."""
    Hq, Hkv, D, dt = shape
    for cu, T in metadata_cases():
        cu_d = torch.as_tensor(cu, device=DEV)
        for pos_offset in (0, 77):
            o = P.make_options(pos_offset=pos_offset)
            rows = P.rope_qk_norm_tile_positions(cu_d, T, Hq, Hkv, D, dt, backward, o)
            # q's tiles come first, then k's: each tensor's rows cover every
            # token (q's tile count is that of the same call without k)
            nq = P.rope_qk_norm_tile_positions(cu_d, T, Hq, 0, D, dt, backward, o).shape[0]
            what = f"norm {'bwd' if backward else 'fwd'} {shape} T={T} nseq={cu.size - 1} offset={pos_offset}"
            check_rows(rows[:nq], cu, T, pos_offset, what + " q")
            check_rows(rows[nq:], cu, T, pos_offset, what + " k")


def test_per_token_positions_use_the_tile_code():
    """rope_qk_positions (tiles of 64 whole tokens, no offset) against the oracle."""
    for cu, T in metadata_cases():
        got = P.rope_qk_positions(torch.as_tensor(cu, device=DEV), T).cpu().numpy()
        assert np.array_equal(got, oracle.segment_positions(cu, T)), (cu[:6], T)
