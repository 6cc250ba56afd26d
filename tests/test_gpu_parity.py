"""HIP path vs the fp64 oracle, element by element, through the C ABI (needs an MI355X).

Every workload is compared element by element in full: the small ones in
one piece, the large model-shaped ones at their full sizes, in the launch
configuration the benchmark times, chunk by chunk on a host thread pool.
"""

import numpy as np
import pytest
import torch

import oracle
import packed_varlen_rotary_amd as P
import workloads as W
from tests import oracle_pins
from tests.gpu_util import MIN_EXACT_FRACTION_AT_SCALE, bits16, check_against, check_every_element, f64, sample_tokens

pytestmark = pytest.mark.gpu

DEV = "cuda"


def cu_dev(cu):
    return torch.as_tensor(np.asarray(cu, dtype=np.int32), device=DEV)


def run(direction, q, k, cu, theta):
    (P.rope_qk_fwd if direction == 1 else P.rope_qk_bwd)(q, k, cu_dev(cu) if not torch.is_tensor(cu) else cu, theta)


def full_check(w, direction, salt=0):
    names = ("q", "k") if direction == 1 else ("dq", "dk")
    t = W.make_tensors(w, names, device=DEV, salt=salt)
    x = {n: f64(t[n]) for n in names}
    run(direction, t[names[0]], t[names[1]], w.cu_seqlens, w.theta)
    torch.cuda.synchronize()
    stats = {}
    for n in names:
        ref = oracle.rope(x[n], w.cu_seqlens, w.theta, direction)
        stats[n] = check_against(t[n], ref, f"{w.name} {n}")
    return stats


def test_positions_bit_exact():
    cases = [(np.array(cu), T) for cu, T in oracle_pins.POSITION_CASES]
    for cfg in (1, 2, 3, 4, 5):
        w = W.make_workload(cfg)
        cases.append((w.cu_seqlens, w.T))
    rng = np.random.default_rng(7)
    many = np.sort(rng.integers(0, 5000, size=3000))  # thousands of segments, many empty
    cases.append((np.concatenate([[0], many, [5000]]), 5003))
    for cu, T in cases:
        got = P.rope_qk_positions(cu_dev(cu), T).cpu().numpy()
        assert np.array_equal(got, oracle.segment_positions(cu, T)), cu[:8]


@pytest.mark.parametrize("direction", [1, -1])
def test_tiny_fp32(direction):
    s = full_check(W.make_workload(1), direction)
    print(s)


@pytest.mark.parametrize("direction", [1, -1])
def test_qwen25_graded_row(direction):
    s = full_check(W.make_workload(2), direction)
    print(s)
    for v in s.values():
        assert v["exact_fraction"] == 1.0, v  # one correctly rounded float64 result


def test_qwen25_every_bfd_row():
    for r in range(W.qwen25_05b_row_count()):
        w = W.make_workload(2, row=r)
        full_check(w, 1, salt=r + 1)


@pytest.mark.parametrize("cfg", [3, 4, 5])
@pytest.mark.parametrize("direction", [1, -1])
def test_model_shapes_every_element(cfg, direction):
    """The Qwen3-8B, Qwen3-32B and 524,288-token workloads at full size, in
    the launch configuration the benchmark times: every element of q and k
    (2.7e9 of them in the long context) against the oracle, bit for bit."""
    w = W.make_workload(cfg)
    names = ("q", "k") if direction == 1 else ("dq", "dk")
    t = W.make_tensors(w, names, device=DEV)
    before = {n: t[n].clone() for n in names}
    run(direction, t[names[0]], t[names[1]], w.cu_seqlens, w.theta)
    torch.cuda.synchronize()
    for n in names:
        s = check_every_element(before[n], t[n], w.cu_seqlens, w.theta, direction, f"{w.name} {n}")
        print(n, s, flush=True)
        assert s["exact_fraction"] >= MIN_EXACT_FRACTION_AT_SCALE, s
    del t, before
    torch.cuda.empty_cache()


def test_long_context_fused_qkv_view():
    """Long-context shapes as q/k views into one [T, Hq + 2 Hkv, D] buffer:
    element offsets pass 2^31.  Forward, then backward on the forward's
    output, each checked on every element of q and k; v is never touched."""
    w = W.make_workload(5)
    H = w.Hq + 2 * w.Hkv
    buf = W.randn((w.T, H, w.D), "bf16", seed=5005, device=DEV)
    assert (w.T - 1) * H * w.D > 2 ** 31  # the last tokens of q sit past element 2^31
    q = buf[:, : w.Hq]
    k = buf[:, w.Hq: w.Hq + w.Hkv]
    v_before = buf[:, w.Hq + w.Hkv:].clone()
    for direction, fn in ((1, P.rope_qk_fwd), (-1, P.rope_qk_bwd)):
        xq, xk = q.clone(), k.clone()
        fn(q, k, cu_dev(w.cu_seqlens), w.theta)
        torch.cuda.synchronize()
        for name, x, y in (("q", xq, q), ("k", xk, k)):
            s = check_every_element(x, y, w.cu_seqlens, w.theta, direction, f"fused {name} dir {direction}")
            print(name, direction, s, flush=True)
            assert s["exact_fraction"] >= MIN_EXACT_FRACTION_AT_SCALE, s
        del xq, xk
    assert torch.equal(buf[:, w.Hq + w.Hkv:], v_before)  # v is never touched
    del buf, v_before
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# shapes, layouts and edge cases
# ---------------------------------------------------------------------------

SHAPES = [
    # (T, Hq, Hkv, D, dtype, cu)
    (97, 3, 1, 16, "bf16", [0, 1, 50, 97]),
    (300, 5, 5, 80, "bf16", [0, 120, 120, 290]),  # 5 chunks per half head, empty segment, tail outside
    (257, 7, 3, 96, "bf16", [0, 257]),
    (64, 2, 2, 256, "bf16", [0, 10, 64]),
    (33, 4, 2, 512, "bf16", [0, 33]),
    (130, 128, 16, 128, "bf16", [0, 60, 130]),  # more than one pass of tasks per token
    (513, 7, 1, 32, "bf16", [0, 100, 513]),  # half row of 2 chunks: chunk tasks, partner 2 lanes away
    (211, 5, 1, 64, "bf16", [4, 90, 90, 200]),  # 4 chunks, 48 tasks per token (general addresses), outside at both ends
    (77, 2, 3, 16, "bf16", [0, 0, 30, 77]),  # half row of 1 chunk, 10 tasks per token, empty first segment
    (129, 2, 2, 48, "bf16", [0, 64, 129]),  # 3 chunks per half row: chunk-pair tasks
    (300, 5, 3, 32, "fp32", [0, 17, 300]),  # fp32 half row of 4 chunks
    (77, 3, 2, 16, "fp32", [0, 77]),  # fp32 half row of 2 chunks
    (1000, 6, 2, 8, "fp32", [0, 999, 1000]),
    (511, 9, 1, 136, "fp32", [3, 200, 480]),
    (40, 1, 1, 2 * 4, "fp32", [0, 40]),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"T{s[0]}_H{s[1]}x{s[2]}_D{s[3]}_{s[4]}")
@pytest.mark.parametrize("direction", [1, -1])
def test_shapes(shape, direction):
    T, Hq, Hkv, D, dt, cu = shape
    q = W.randn((T, Hq, D), dt, seed=T * 7 + D, device=DEV)
    k = W.randn((T, Hkv, D), dt, seed=T * 11 + D, device=DEV)
    xq, xk = f64(q), f64(k)
    run(direction, q, k, cu, 1e4)
    torch.cuda.synchronize()
    check_against(q, oracle.rope(xq, cu, 1e4, direction), "q")
    check_against(k, oracle.rope(xk, cu, 1e4, direction), "k")



def _random_chunk_task_cases(n=24, seed=2026):
    """Seeded random shapes whose half rows are 1, 2 or 4 chunks (the chunk
    tasks, where the two lanes of a row's chunk pair split its element
    pairs): every storage type, 1-20 q heads and 0-5 k heads (token task
    counts that divide 256 and that do not), 1-699 tokens, and packings with
    empty segments and tokens outside every sequence at either end."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dt = ("bf16", "fp16", "fp32")[i % 3]
        D = int(rng.choice([8, 16, 32] if dt == "fp32" else [16, 32, 64]))
        Hq, Hkv, T = int(rng.integers(1, 21)), int(rng.integers(0, 6)), int(rng.integers(1, 700))
        lo = int(rng.integers(0, min(T, 3) + 1))
        hi = T - int(rng.integers(0, min(T - lo, 3) + 1))
        cu = [lo] + sorted(int(c) for c in rng.integers(lo, hi + 1, size=int(rng.integers(1, 12))))
        cases.append((T, Hq, Hkv, D, dt, cu, float(rng.choice([1e4, 1e6]))))
    return cases


@pytest.mark.parametrize("case", _random_chunk_task_cases(), ids=lambda c: f"T{c[0]}_H{c[1]}x{c[2]}_D{c[3]}_{c[4]}")
@pytest.mark.parametrize("direction", [1, -1])
def test_chunk_tasks_random_shapes(case, direction):
    T, Hq, Hkv, D, dt, cu, theta = case
    q = W.randn((T, Hq, D), dt, seed=T * 13 + Hq, device=DEV)
    k = W.randn((T, Hkv, D), dt, seed=T * 17 + Hkv + 1, device=DEV)
    xq, xk = f64(q), f64(k)
    run(direction, q, k, cu, theta)
    torch.cuda.synchronize()
    for name, out, x in (("q", q, xq), ("k", k, xk)):
        st = check_against(out, oracle.rope(x, cu, theta, direction), name)
        if dt != "fp32":
            assert st["exact_fraction"] == 1.0, (name, st)

def test_tokens_outside_sequences_untouched():
    T, cu = 256, [5, 100, 100, 200]
    q = W.randn((T, 4, 64), "bf16", seed=1, device=DEV)
    k = W.randn((T, 2, 64), "bf16", seed=2, device=DEV)
    q0, k0 = q.clone(), k.clone()
    run(1, q, k, cu, 1e6)
    torch.cuda.synchronize()
    for a, b in ((q, q0), (k, k0)):
        assert torch.equal(a[:5], b[:5]) and torch.equal(a[200:], b[200:])
        assert not torch.equal(a[6:100], b[6:100])


def test_head_major_view_in_place():
    """A [H, T, D] buffer seen as [T, H, D]: no clone or transposed copy is needed."""
    T, Hq, Hkv, D = 300, 6, 2, 64
    bq = W.randn((Hq, T, D), "bf16", seed=3, device=DEV)
    bk = W.randn((Hkv, T, D), "bf16", seed=4, device=DEV)
    q, k = bq.permute(1, 0, 2), bk.permute(1, 0, 2)
    assert not q.is_contiguous()
    xq, xk = f64(q), f64(k)
    cu = [0, 100, 300]
    run(1, q, k, cu, 1e6)
    torch.cuda.synchronize()
    check_against(q, oracle.rope(xq, cu, 1e6, 1), "q head-major")
    check_against(k, oracle.rope(xk, cu, 1e6, 1), "k head-major")


@pytest.mark.parametrize("D", [16, 32, 64, 128])
def test_rows_off_cache_line(D):
    """Rows that start 16 bytes past a 128-byte line (a fused buffer with an odd offset)."""
    T, Hq, Hkv = 203, 5, 3
    raw = W.randn((T * (Hq + Hkv) * D + 8,), "bf16", seed=D, device=DEV)
    qk = raw[8:].view(T, Hq + Hkv, D)
    q, k = qk[:, :Hq], qk[:, Hq:]
    assert q.data_ptr() % 128 == 16
    xq, xk = f64(q), f64(k)
    cu = [0, 1, 90, 203]
    run(1, q, k, cu, 1e4)
    torch.cuda.synchronize()
    check_against(q, oracle.rope(xq, cu, 1e4, 1), f"q D{D}")
    check_against(k, oracle.rope(xk, cu, 1e4, 1), f"k D{D}")


def test_no_kv_heads():
    T, D = 50, 64
    q = W.randn((T, 4, D), "bf16", seed=5, device=DEV)
    k = torch.empty((T, 0, D), dtype=torch.bfloat16, device=DEV)
    xq = f64(q)
    run(1, q, k, [0, 20, 50], 1e4)
    torch.cuda.synchronize()
    check_against(q, oracle.rope(xq, [0, 20, 50], 1e4, 1), "q only")


def test_guard_bands_intact():
    """The kernel writes nothing outside the q/k rows it owns."""
    T, Hq, Hkv, D = 777, 14, 2, 64
    nq, nk = T * Hq * D, T * Hkv * D
    pad = 4096
    sentinel = torch.full((nq + nk + 3 * pad,), -12345, dtype=torch.int16, device=DEV)
    raw = sentinel.view(torch.bfloat16)
    src = W.randn((nq + nk,), "bf16", seed=9, device=DEV)
    raw[pad: pad + nq] = src[:nq]
    raw[2 * pad + nq: 2 * pad + nq + nk] = src[nq:]
    q = raw[pad: pad + nq].view(T, Hq, D)
    k = raw[2 * pad + nq: 2 * pad + nq + nk].view(T, Hkv, D)
    run(1, q, k, [0, 300, T], 1e6)
    torch.cuda.synchronize()
    g = sentinel.cpu().numpy()
    assert np.all(g[:pad] == -12345)
    assert np.all(g[pad + nq: 2 * pad + nq] == -12345)
    assert np.all(g[2 * pad + nq + nk:] == -12345)


def test_position_zero_is_identity_and_packed_equals_unpacked():
    w = W.make_workload(2)
    t = W.make_tensors(w, ("q", "k"), device=DEV)
    packed_q, packed_k = t["q"].clone(), t["k"].clone()
    run(1, packed_q, packed_k, w.cu_seqlens, w.theta)
    starts = torch.as_tensor(w.cu_seqlens[:-1].astype(np.int64), device=DEV)
    assert torch.equal(packed_q.index_select(0, starts), t["q"].index_select(0, starts))
    assert torch.equal(packed_k.index_select(0, starts), t["k"].index_select(0, starts))
    # each sequence on its own, as an unpacked batch of one
    for s in range(w.nseq):
        a, b = int(w.cu_seqlens[s]), int(w.cu_seqlens[s + 1])
        q1, k1 = t["q"][a:b].clone(), t["k"][a:b].clone()
        run(1, q1, k1, [0, b - a], w.theta)
        assert torch.equal(q1, packed_q[a:b]) and torch.equal(k1, packed_k[a:b]), s
    torch.cuda.synchronize()


def test_backward_undoes_forward_and_is_deterministic():
    w = W.make_workload(2)
    t = W.make_tensors(w, ("q", "k"), device=DEV)
    q, k = t["q"].clone(), t["k"].clone()
    run(1, q, k, w.cu_seqlens, w.theta)
    q2, k2 = t["q"].clone(), t["k"].clone()
    run(1, q2, k2, w.cu_seqlens, w.theta)
    assert torch.equal(q, q2) and torch.equal(k, k2)  # run-to-run bit-exact
    run(-1, q, k, w.cu_seqlens, w.theta)
    torch.cuda.synchronize()
    # bf16 rounding moves each element by at most 2^-8 of its magnitude.  The
    # forward rounding error e has |e| <= 2^-8 |x| over the pair (rotations keep
    # norms), the rotated-back error is R^T e, and the final rounding adds at most
    # 2^-8 (|x_i| + |e|), so |z_i - x_i| <= 2^-8 |x| (2 + 2^-8) with |x| the pair norm.
    # A per-element ulp bound would not hold: a small element next to a large
    # partner inherits the partner's rounding error.
    for a, b in ((q, t["q"]), (k, t["k"])):
        x, z = f64(b), f64(a)
        half = x.shape[-1] // 2
        norm = np.sqrt(x[..., :half] ** 2 + x[..., half:] ** 2)
        norm = np.concatenate([norm, norm], axis=-1)
        assert np.all(np.abs(z - x) <= 2.0 ** -8 * (2 + 2.0 ** -8) * norm)


def test_fp32_backward_undoes_forward():
    w = W.make_workload(1)
    t = W.make_tensors(w, ("q", "k"), device=DEV)
    q, k = t["q"].clone(), t["k"].clone()
    run(1, q, k, w.cu_seqlens, w.theta)
    run(-1, q, k, w.cu_seqlens, w.theta)
    torch.cuda.synchronize()
    assert (q - t["q"]).abs().max().item() <= 2e-6 and (k - t["k"]).abs().max().item() <= 2e-6


def test_side_stream_and_binding_errors():
    w = W.make_workload(1)
    t = W.make_tensors(w, ("q", "k"), device=DEV)
    x = f64(t["q"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        P.rope_qk_fwd(t["q"], t["k"], cu_dev(w.cu_seqlens), w.theta)
    s.synchronize()
    check_against(t["q"], oracle.rope(x, w.cu_seqlens, w.theta, 1), "side stream")
    odd = torch.zeros(8, 2, 66, dtype=torch.bfloat16, device=DEV)[:, :, 1:65]  # 2-byte misaligned view
    odd_k = torch.zeros(8, 1, 66, dtype=torch.bfloat16, device=DEV)[:, :, 1:65]
    with pytest.raises(P.RopeQKError) as e:
        P.rope_qk_fwd(odd, odd_k, cu_dev([0, 8]), 1e4)
    assert e.value.status == -4
    with pytest.raises(P.RopeQKError) as e:  # q and k sharing memory
        P.rope_qk_fwd(t["q"], t["q"][:, :2], cu_dev(w.cu_seqlens), w.theta)
    assert e.value.status == -7


@pytest.mark.parametrize("offset", [0, 2 ** 31 - 1 - 600])
def test_short_sequences_and_large_positions(offset):
    """Few heads at D = 64 and 32, so a tile's table spans many tokens;
    sequences of 1 to 5 tokens put many boundaries inside each tile;
    positions up to 2^31 - 2, where an angle's float64 ulp is largest.  Every
    element exact against the oracle."""
    rng = np.random.default_rng(77)
    T = 600
    lengths = np.concatenate([[300], rng.integers(1, 6, size=200)])  # segment 0 carries the offset
    cu = np.concatenate([[0], np.cumsum(lengths)])
    cu = cu[cu <= T]
    for D, Hq, Hkv in ((64, 2, 1), (32, 1, 1)):
        q = W.randn((T, Hq, D), "bf16", seed=D, device=DEV)
        k = W.randn((T, Hkv, D), "bf16", seed=D + 1, device=DEV)
        xq, xk = f64(q), f64(k)
        P.rope_qk_fwd(q, k, cu_dev(cu), 1e4, pos_offset=offset)
        torch.cuda.synchronize()
        for got, x in ((q, xq), (k, xk)):
            s = check_against(got, oracle.rope(x, cu, 1e4, 1, pos_offset=offset), f"D{D}")
            assert s["exact_fraction"] == 1.0, s


@pytest.mark.parametrize("delta", [1, 4097, 500_000])
def test_scores_depend_only_on_relative_position(delta):
    """The property that makes the rotation a relative position encoding: the
    score <f(q, m), f(k, n)> is the same when every position moves by delta.
    fp32 q and k (GQA, 4 q heads per k head) rotated at positions 0..S-1 and
    again, from fresh copies, at delta..delta+S-1 (pos_offset); every (m, n)
    score of every head, in float64 from the stored fp32 outputs, agrees
    within 1e-5 of |q_m| |k_n| (each output element carries one fp32 rounding,
    the angles one float64 rounding)."""
    S, Hq, Hkv, D = 96, 8, 2, 64
    q = W.randn((S, Hq, D), "fp32", seed=delta, device=DEV)
    k = W.randn((S, Hkv, D), "fp32", seed=delta + 1, device=DEV)
    cu = cu_dev([0, S])
    q0, k0, q1, k1 = q.clone(), k.clone(), q.clone(), k.clone()
    P.rope_qk_fwd(q0, k0, cu, 1e4)
    P.rope_qk_fwd(q1, k1, cu, 1e4, pos_offset=delta)
    torch.cuda.synchronize()
    g = Hq // Hkv
    for a, b in ((q0, k0), (q1, k1)):
        assert torch.isfinite(a).all() and torch.isfinite(b).all()

    def scores(qr, kr):  # [Hq, S(m), S(n)] in float64, each q head against its k head
        qh = f64(qr).transpose(1, 0, 2)
        kh = np.repeat(f64(kr), g, axis=1).transpose(1, 2, 0)
        return qh @ kh

    s0, s1 = scores(q0, k0), scores(q1, k1)
    qn = np.linalg.norm(f64(q), axis=-1).T[:, :, None]
    kn = np.repeat(np.linalg.norm(f64(k), axis=-1), g, axis=1).T[:, None, :]
    err = np.abs(s0 - s1) / (qn * kn)
    assert float(err.max()) <= 1e-5, float(err.max())
    # and the positions did move: the rotated tensors themselves differ
    assert not torch.equal(q0, q1)
