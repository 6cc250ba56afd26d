"""Per-head RMSNorm + rotation through the C ABI vs the fp64 oracle (needs an MI355X).

Forward: every row shape (2 to 64 chunks of 16 bytes per head) in bf16, fp16
and fp32, in place and out of place, with the rotation options.  Backward:
dx element by element like the forward; the weight gradients against the
oracle's float64 sums to within about one float32 ulp, and run-to-run
identical.  The Qwen3-8B-shaped batch and the 524,288-token context run at
full size, every element of every output checked, the weight gradients
against the oracle summed over every token.
"""

import numpy as np
import pytest
import torch

import oracle
import packed_varlen_rotary_amd as P
import workloads as W
from tests.gpu_util import MIN_EXACT_FRACTION_AT_SCALE, check_against, check_chunks, f64

pytestmark = pytest.mark.gpu

DEV = "cuda"
EPS = 1e-6
LLAMA3 = dict(factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0, original_max_position=8192.0)


def cu_dev(cu):
    return torch.as_tensor(np.asarray(cu, dtype=np.int32), device=DEV)


def weights(D, seed):
    """A norm weight near 1, like trained q/k norm weights (float32)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return (1.0 + 0.25 * torch.randn(D, generator=g)).float().to(DEV)


def oracle_opts(opts):
    return dict(pos_offset=opts.get("pos_offset", 0), pairing="interleaved" if opts.get("interleaved") else "half",
                scaling=opts.get("llama3"), freq_precision="fp32" if opts.get("freq_fp32") else "fp64")


def w64(w):
    return w.detach().cpu().double().numpy()


def check_dw(got, ref, S, what):
    """float32 weight gradient vs the oracle's float64 sum: half an fp32 ulp of
    the value, plus 1e-11 of the sum of |terms| for float64 summation order."""
    got = got.detach().cpu().double().numpy()
    err = np.abs(got - ref)
    bound = 2.0 ** -24 * np.abs(ref) + 1e-11 * S + 1e-30
    assert np.all(err <= bound), f"{what}: worst {np.max(err / bound)} of the bound"


def dw_terms(dy, x, w, cu, theta, o):
    """sum over normalised heads of |dn_j x_j r|: the scale of the weight-gradient sums."""
    T = x.shape[0]
    inside = oracle.segment_positions(cu, T, o["pos_offset"]) >= 0
    dn = oracle.rope(dy, cu, theta, -1, **o)
    _, r = oracle.rms_norm(x, w, EPS)
    return np.sum(np.abs(dn * x * r[..., None])[inside], axis=(0, 1))


SHAPES = [
    # T, Hq, Hkv, D, dtype (chunks per head = D * size / 16)
    (300, 6, 2, 128, "bf16"),  # 16
    (257, 5, 3, 64, "bf16"),  # 8
    (129, 4, 2, 256, "bf16"),  # 32
    (65, 3, 2, 512, "bf16"),  # 64: a row fills a wave
    (400, 7, 1, 16, "bf16"),  # 2
    (300, 4, 4, 32, "bf16"),  # 4
    (300, 6, 2, 64, "fp32"),  # 16
    (200, 3, 1, 128, "fp32"),  # 32
    (500, 5, 3, 8, "fp32"),  # 2
    (150, 2, 2, 256, "fp32"),  # 64
    (300, 6, 2, 128, "fp16"),
    (257, 5, 3, 64, "fp16"),
]


def run_fwd(q, k, wq, wk, cu, theta, out_of_place, **opts):
    xq, xk = f64(q), f64(k)
    q0, k0 = q.clone(), k.clone()
    if out_of_place:
        qo, ko = torch.full_like(q, 3.0), torch.full_like(k, 3.0)
    else:
        qo, ko = q, k
    P.rope_qk_norm_fwd(q, k, wq, wk, EPS, cu_dev(cu), theta, qo, ko, **opts)
    torch.cuda.synchronize()
    o = oracle_opts(opts)
    rq, _ = oracle.norm_rope(xq, w64(wq), EPS, cu, theta, **o)
    rk, _ = oracle.norm_rope(xk, w64(wk), EPS, cu, theta, **o)
    sq = check_against(qo, rq, f"q {opts}")
    sk = check_against(ko, rk, f"k {opts}")
    if out_of_place:
        assert torch.equal(q, q0) and torch.equal(k, k0)  # inputs untouched
    return sq, sk


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"T{s[0]}_H{s[1]}x{s[2]}_D{s[3]}_{s[4]}")
@pytest.mark.parametrize("out_of_place", [False, True], ids=["inplace", "outofplace"])
def test_norm_fwd_shapes(shape, out_of_place):
    T, Hq, Hkv, D, dt = shape
    q = W.randn((T, Hq, D), dt, seed=T + D, device=DEV)
    k = W.randn((T, Hkv, D), dt, seed=T + D + 1, device=DEV)
    cu = [0, 1, T // 3, T // 3, T - 5]  # a 1-token sequence, an empty one, 5 tokens outside
    sq, sk = run_fwd(q, k, weights(D, D), weights(D, D + 1), cu, 1e4, out_of_place)
    if dt != "fp32":
        assert sq["exact_fraction"] == 1.0 and sk["exact_fraction"] == 1.0, (sq, sk)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("opts", [dict(interleaved=True), dict(pos_offset=123456, llama3=LLAMA3),
                                  dict(freq_fp32=True, pos_offset=500000),
                                  dict(interleaved=True, pos_offset=77, llama3=LLAMA3, freq_fp32=True)],
                         ids=["interleaved", "offset_llama3", "fp32_angles", "everything"])
def test_norm_fwd_options(dt, opts):
    T, Hq, Hkv, D = 300, 6, 2, 128
    q = W.randn((T, Hq, D), dt, seed=11, device=DEV)
    k = W.randn((T, Hkv, D), dt, seed=12, device=DEV)
    run_fwd(q, k, weights(D, 5), weights(D, 6), [0, 100, 100, 290], 5e5, True, **opts)


def run_bwd(T, Hq, Hkv, D, dt, cu, theta, seed, in_place, zero_w=None, **opts):
    """zero_w: {"q": [elements], "k": [...]} set to exactly 0 in that tensor's weights."""
    q = W.randn((T, Hq, D), dt, seed=seed, device=DEV)
    k = W.randn((T, Hkv, D), dt, seed=seed + 1, device=DEV)
    dyq = W.randn((T, Hq, D), dt, seed=seed + 2, device=DEV)
    dyk = W.randn((T, Hkv, D), dt, seed=seed + 3, device=DEV)
    wq, wk = weights(D, seed + 4), weights(D, seed + 5)
    for name, w in (("q", wq), ("k", wk)):
        for j in (zero_w or {}).get(name, []):
            w[j] = 0.0
    xq, xk, gq, gk = f64(q), f64(k), f64(dyq), f64(dyk)
    if in_place:
        dq, dk = dyq, dyk
    else:
        dq, dk = torch.full_like(q, 5.0), torch.full_like(k, 5.0)
    dq, dk, dwq, dwk = P.rope_qk_norm_bwd(dyq, dyk, q, k, wq, wk, EPS, cu_dev(cu), theta, dq, dk, **opts)
    torch.cuda.synchronize()
    o = oracle_opts(opts)
    out = {}
    for name, dx, dw, x, g, w in (("q", dq, dwq, xq, gq, wq), ("k", dk, dwk, xk, gk, wk)):
        rdx, rdw = oracle.norm_rope_bwd(g, x, w64(w), EPS, cu, theta, **o)
        out[name] = check_against(dx, rdx, f"d{name} {opts}")
        check_dw(dw, rdw, dw_terms(g, x, w64(w), cu, theta, o), f"dw{name} {opts}")
    return out


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"T{s[0]}_H{s[1]}x{s[2]}_D{s[3]}_{s[4]}")
def test_norm_bwd_shapes(shape):
    T, Hq, Hkv, D, dt = shape
    cu = [0, 1, T // 3, T // 3, T - 5]
    s = run_bwd(T, Hq, Hkv, D, dt, cu, 1e4, seed=7 * T + D, in_place=True)
    if dt != "fp32":
        assert s["q"]["exact_fraction"] == 1.0 and s["k"]["exact_fraction"] == 1.0, s


@pytest.mark.parametrize("opts", [dict(), dict(interleaved=True), dict(pos_offset=4096, llama3=LLAMA3, freq_fp32=True)],
                         ids=["plain", "interleaved", "offset_llama3_fp32"])
def test_norm_bwd_out_of_place_and_options(opts):
    run_bwd(700, 8, 2, 128, "bf16", [3, 100, 100, 620, 690], 5e5, seed=91, in_place=False, **opts)


@pytest.mark.parametrize("which", ["q", "k"])
@pytest.mark.parametrize("shape", [(300, 6, 2, 128, "bf16", {}), (257, 5, 3, 64, "fp16", {}),
                                   (300, 6, 2, 64, "fp32", {}), (300, 6, 2, 128, "bf16", dict(interleaved=True))],
                         ids=lambda s: f"T{s[0]}_H{s[1]}x{s[2]}_D{s[3]}_{s[4]}_{'il' if s[5] else 'half'}")
def test_norm_bwd_zero_weights(shape, which):
    """With every weight finite and nonzero the backward folds the weights
    into its cos/sin tables (the rotation of dy then gives w dn directly, and
    the weight-gradient sums of w dn x r are divided by w at the end).  A
    weight of exactly zero, in q's vector or in k's, rules that out: the
    kernel then rotates with unit weights and multiplies by w.  Zeros on an
    element, on its rotation partner and on one more: dx bit-exact (g is 0
    there) and the weight gradients, nonzero where w is 0, against the oracle."""
    T, Hq, Hkv, D, dt, opts = shape
    zeros = [0, 1 if opts.get("interleaved") else D // 2, 5]
    s = run_bwd(T, Hq, Hkv, D, dt, [0, 1, T // 3, T // 3, T - 5], 1e4, seed=D + T, in_place=False,
                zero_w={which: zeros}, **opts)
    if dt != "fp32":
        assert s["q"]["exact_fraction"] == 1.0 and s["k"]["exact_fraction"] == 1.0, s


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
def test_norm_bwd_weights_of_every_magnitude(dt):
    """The folded backward forms g = w dn in its tables and divides the
    weight-gradient sums of w dn x r by w at the end: weights from 1e-20 to
    1e20 in size in bf16, of either sign (1e-3 to 1e3 for fp16, whose
    outputs must stay in range, and for fp32, checked against the scaled
    fp32 bound), against the oracle's unfolded float64 sums."""
    T, Hq, Hkv, D = 300, 6, 2, 128
    lo, hi = (-3.0, 3.0) if dt != "bf16" else (-20.0, 20.0)
    g = torch.Generator(device="cpu")
    g.manual_seed(81)
    mags = 10.0 ** (lo + (hi - lo) * torch.rand(2, D, generator=g, dtype=torch.float64))
    signs = torch.where(torch.rand(2, D, generator=g) < 0.5, -1.0, 1.0).double()
    ws = (mags * signs).float().to(DEV)
    cu = [0, 1, 120, 120, 296]
    q = W.randn((T, Hq, D), dt, seed=82, device=DEV)
    k = W.randn((T, Hkv, D), dt, seed=83, device=DEV)
    dyq = W.randn((T, Hq, D), dt, seed=84, device=DEV)
    dyk = W.randn((T, Hkv, D), dt, seed=85, device=DEV)
    dq, dk, dwq, dwk = P.rope_qk_norm_bwd(dyq.clone(), dyk.clone(), q, k, ws[0], ws[1], EPS, cu_dev(cu), 1e4)
    torch.cuda.synchronize()
    o = oracle_opts({})
    for name, dx, dw, x, dy, w in (("q", dq, dwq, q, dyq, ws[0]), ("k", dk, dwk, k, dyk, ws[1])):
        rdx, rdw = oracle.norm_rope_bwd(f64(dy), f64(x), w64(w), EPS, cu, 1e4, **o)
        if dt == "fp32":  # the fp32 bound of the unit-scale tests, scaled by the outputs' size
            err = np.abs(f64(dx) - rdx)
            scale = max(1.0, float(np.abs(rdx).max()))
            assert float(err.max()) <= 1e-5 * scale, f"d{name}: {err.max()} at scale {scale}"
        else:
            st = check_against(dx, rdx, f"d{name} weights 1e{lo:+.0f}..1e{hi:+.0f}")
            assert st["exact_fraction"] == 1.0, st
        check_dw(dw, rdw, dw_terms(f64(dy), f64(x), w64(w), cu, 1e4, o), f"dw{name} weights of every magnitude")


def test_norm_bwd_tensor_without_heads():
    """k with no heads: its weight vector (all zeros here) plays no part, so
    q's backward still folds its weights; q's results match the oracle and
    k's weight gradient is zero."""
    T, Hq, D = 300, 6, 128
    cu = [0, 1, 100, 100, 295]
    q = W.randn((T, Hq, D), "bf16", seed=61, device=DEV)
    dyq = W.randn((T, Hq, D), "bf16", seed=62, device=DEV)
    k = torch.empty((T, 0, D), dtype=torch.bfloat16, device=DEV)
    wq, wk = weights(D, 63), torch.zeros(D, dtype=torch.float32, device=DEV)
    dq, dk, dwq, dwk = P.rope_qk_norm_bwd(dyq.clone(), k.clone(), q, k, wq, wk, EPS, cu_dev(cu), 1e4)
    torch.cuda.synchronize()
    o = oracle_opts({})
    rdx, rdw = oracle.norm_rope_bwd(f64(dyq), f64(q), w64(wq), EPS, cu, 1e4, **o)
    s = check_against(dq, rdx, "dq without k heads")
    assert s["exact_fraction"] == 1.0, s
    check_dw(dwq, rdw, dw_terms(f64(dyq), f64(q), w64(wq), cu, 1e4, o), "dwq without k heads")
    assert torch.equal(dwk, torch.zeros_like(dwk))


@pytest.mark.parametrize("shape", [(2000, 6, 2, 128, "bf16"), (1500, 1, 1, 64, "bf16"), (900, 40, 8, 128, "fp16"),
                                   (1200, 3, 3, 32, "fp32")],
                         ids=lambda s: f"T{s[0]}_H{s[1]}x{s[2]}_D{s[3]}_{s[4]}")
def test_norm_many_short_sequences(shape):
    """Hundreds of sequences of 0 to 7 tokens (empty ones included) after a
    long first one, then tokens outside: tiles start and end inside
    sequences, hold several boundaries, and the backward's workgroups step
    through many boundaries in their runs of tiles.  Forward and backward
    against the oracle."""
    T, Hq, Hkv, D, dt = shape
    rng = np.random.default_rng(T + Hq)
    lengths = np.concatenate([[137], rng.integers(0, 8, size=T)])
    cu = np.concatenate([[0], np.cumsum(lengths)])
    cu = cu[cu <= T - 9]  # the last 9+ tokens lie outside
    q = W.randn((T, Hq, D), dt, seed=T, device=DEV)
    k = W.randn((T, Hkv, D), dt, seed=T + 1, device=DEV)
    sq, sk = run_fwd(q, k, weights(D, 1), weights(D, 2), cu, 1e4, True)
    s = run_bwd(T, Hq, Hkv, D, dt, cu, 1e4, seed=T + 2, in_place=False)
    if dt != "fp32":
        for r in (sq, sk, s["q"], s["k"]):
            assert r["exact_fraction"] == 1.0, r


def test_norm_bwd_long_runs_of_tiles():
    """Enough tiles (12,667) that each backward workgroup takes a run of about
    eight (1,583 workgroups), over thousands of sequences of 0 to 7 tokens: the cursor into
    cu_seqlens steps across many boundaries inside a run and from tile to
    tile, and one run crosses from q's tiles to k's.  dx bit-exact, dw to the
    oracle's sums."""
    T, Hq, Hkv, D = 40000, 8, 2, 128
    rng = np.random.default_rng(4242)
    lengths = np.concatenate([[137], rng.integers(0, 8, size=T)])
    cu = np.concatenate([[0], np.cumsum(lengths)])
    cu = cu[cu <= T - 9]
    s = run_bwd(T, Hq, Hkv, D, "bf16", cu, 1e4, seed=4243, in_place=True)
    assert s["q"]["exact_fraction"] == 1.0 and s["k"]["exact_fraction"] == 1.0, s


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_norm_strided_views(dt):
    """q and k as views into fused QKV buffers (token stride (Hq + 2 Hkv) D,
    so rows are not evenly spaced), outputs and gradients both contiguous and
    strided: the general (token, head) addressing, against the oracle."""
    T, Hq, Hkv, D = 400, 6, 2, 128
    cu = [0, 3, 150, 150, 391]
    W3 = Hq + 2 * Hkv
    qkv = W.randn((T, W3, D), dt, seed=51, device=DEV)
    gqkv = W.randn((T, W3, D), dt, seed=52, device=DEV)
    q, k = qkv[:, :Hq], qkv[:, Hq:Hq + Hkv]
    gq, gk = gqkv[:, :Hq], gqkv[:, Hq:Hq + Hkv]
    assert q.stride(0) == W3 * D and not q.is_contiguous()
    wq, wk = weights(D, 53), weights(D, 54)
    o = oracle_opts({})
    # forward: strided in, contiguous out; then contiguous in, strided out
    yq, yk = torch.empty(T, Hq, D, dtype=q.dtype, device=DEV), torch.empty(T, Hkv, D, dtype=q.dtype, device=DEV)
    P.rope_qk_norm_fwd(q, k, wq, wk, EPS, cu_dev(cu), 1e4, yq, yk)
    out = torch.zeros_like(qkv)
    P.rope_qk_norm_fwd(q.contiguous(), k.contiguous(), wq, wk, EPS, cu_dev(cu), 1e4, out[:, :Hq],
                       out[:, Hq:Hq + Hkv])
    torch.cuda.synchronize()
    for got, x, w in ((yq, q, wq), (yk, k, wk), (out[:, :Hq], q, wq), (out[:, Hq:Hq + Hkv], k, wk)):
        ry, _ = oracle.norm_rope(f64(x), w64(w), EPS, cu, 1e4, **o)
        s = check_against(got, ry, "strided fwd")
        if dt != "fp32":
            assert s["exact_fraction"] == 1.0, s
    # backward: strided dy and x, contiguous dx
    dq, dk, dwq, dwk = P.rope_qk_norm_bwd(gq, gk, q, k, wq, wk, EPS, cu_dev(cu), 1e4,
                                          torch.empty(T, Hq, D, dtype=q.dtype, device=DEV),
                                          torch.empty(T, Hkv, D, dtype=q.dtype, device=DEV))
    torch.cuda.synchronize()
    for dx, dw, x, g, w in ((dq, dwq, q, gq, wq), (dk, dwk, k, gk, wk)):
        rdx, rdw = oracle.norm_rope_bwd(f64(g), f64(x), w64(w), EPS, cu, 1e4, **o)
        s = check_against(dx, rdx, "strided bwd")
        if dt != "fp32":
            assert s["exact_fraction"] == 1.0, s
        check_dw(dw, rdw, dw_terms(f64(g), f64(x), w64(w), cu, 1e4, o), "strided dw")


def test_norm_bwd_outside_tokens_after_nan_tables():
    """The backward's rows of tokens in no sequence enter as zeros; their
    cos/sin entries must not come from whatever an earlier kernel left in LDS.
    A forward with NaN weights first fills the LDS of every compute unit with
    NaN table entries; the backward that follows, on a batch whose tail and
    empty sequences lie outside, must still give finite weight gradients equal
    to the oracle's."""
    T, Hq, Hkv, D, dt = 900, 40, 8, 128, "fp16"
    nan_w = torch.full((D,), float("nan"), dtype=torch.float32, device=DEV)
    xq = W.randn((8192, Hq, D), dt, seed=71, device=DEV)
    xk = W.randn((8192, Hkv, D), dt, seed=72, device=DEV)
    cu_big = cu_dev([0, 8192])
    for _ in range(3):
        P.rope_qk_norm_fwd(xq, xk, nan_w, nan_w, EPS, cu_big, 1e4, torch.empty_like(xq), torch.empty_like(xk))
        cu = [0, 1, 300, 300, 300, 651, 890]  # tokens 890.. lie outside
        run_bwd(T, Hq, Hkv, D, dt, cu, 1e4, seed=73, in_place=False)


def test_norm_nonfinite_rows_outside_sequences():
    """Rows of tokens outside every sequence may hold anything (say, a
    gradient buffer that nothing wrote): NaN and infinities there pass through
    to the outputs bit for bit and change neither the inside rows nor the
    weight gradients, which match the oracle run on finite stand-ins."""
    T, Hq, Hkv, D, dt = 300, 6, 2, 128, "bf16"
    cu = [0, 1, 100, 100, 290]  # tokens 290.. lie outside
    x = {nm: W.randn((T, H, D), dt, seed=s, device=DEV) for nm, H, s in (("q", Hq, 41), ("k", Hkv, 42))}
    gy = {nm: W.randn((T, H, D), dt, seed=s, device=DEV) for nm, H, s in (("q", Hq, 43), ("k", Hkv, 44))}
    bad = torch.tensor([float("nan"), float("inf"), -float("inf"), 1.0], dtype=torch.bfloat16, device=DEV)
    for tns in list(x.values()) + list(gy.values()):
        tail = tns[290:]
        tail.copy_(bad.repeat(tail.numel() // 4 + 1)[: tail.numel()].view_as(tail))
    wq, wk = weights(D, 45), weights(D, 46)
    fin = {nm: f64(v) for nm, v in x.items()}
    fing = {nm: f64(v) for nm, v in gy.items()}
    for arr in list(fin.values()) + list(fing.values()):
        arr[290:] = 0.0  # finite stand-ins: the oracle has no cross-token terms
    yq, yk = torch.empty_like(x["q"]), torch.empty_like(x["k"])
    P.rope_qk_norm_fwd(x["q"], x["k"], wq, wk, EPS, cu_dev(cu), 1e4, yq, yk)
    dq, dk, dwq, dwk = P.rope_qk_norm_bwd(gy["q"].clone(), gy["k"].clone(), x["q"], x["k"], wq, wk, EPS,
                                          cu_dev(cu), 1e4)
    torch.cuda.synchronize()
    o = oracle_opts({})
    for nm, y, dx, dw, w in (("q", yq, dq, dwq, wq), ("k", yk, dk, dwk, wk)):
        ry, _ = oracle.norm_rope(fin[nm], w64(w), EPS, cu, 1e4, **o)
        s = check_against(y[:290], ry[:290], f"fwd {nm} inside")
        assert s["exact_fraction"] == 1.0, s
        assert torch.equal(y[290:].view(torch.int16), x[nm][290:].view(torch.int16))
        rdx, rdw = oracle.norm_rope_bwd(fing[nm], fin[nm], w64(w), EPS, cu, 1e4, **o)
        s = check_against(dx[:290], rdx[:290], f"bwd d{nm} inside")
        assert s["exact_fraction"] == 1.0, s
        assert torch.equal(dx[290:].view(torch.int16), gy[nm][290:].view(torch.int16))
        assert torch.isfinite(dw).all()
        check_dw(dw, rdw, dw_terms(fing[nm], fin[nm], w64(w), cu, 1e4, o), f"dw{nm} with non-finite outside rows")


def test_norm_bwd_is_deterministic():
    T, Hq, Hkv, D = 3000, 16, 4, 128
    q = W.randn((T, Hq, D), "bf16", seed=1, device=DEV)
    k = W.randn((T, Hkv, D), "bf16", seed=2, device=DEV)
    dyq = W.randn((T, Hq, D), "bf16", seed=3, device=DEV)
    dyk = W.randn((T, Hkv, D), "bf16", seed=4, device=DEV)
    wq, wk = weights(D, 1), weights(D, 2)
    cu = cu_dev([0, 1000, 2500, T])
    res = [P.rope_qk_norm_bwd(dyq.clone(), dyk.clone(), q, k, wq, wk, EPS, cu, 1e6) for _ in range(3)]
    torch.cuda.synchronize()
    for r in res[1:]:
        for a, b in zip(res[0], r):
            assert torch.equal(a.view(torch.int16) if a.dtype != torch.float32 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype != torch.float32 else b.view(torch.int32))


def test_norm_bwd_matches_finite_differences_of_the_forward():
    """The GPU backward's dx against a central difference of the GPU forward's
    sum(G * y) along a random direction V (fp32 storage; independent of the
    oracle)."""
    T, Hq, Hkv, D = 64, 4, 2, 64
    q = W.randn((T, Hq, D), "fp32", seed=21, device=DEV)
    k = W.randn((T, Hkv, D), "fp32", seed=22, device=DEV)
    G = W.randn((T, Hq, D), "fp32", seed=23, device=DEV)
    V = W.randn((T, Hq, D), "fp32", seed=24, device=DEV)
    wq, wk = weights(D, 3), weights(D, 4)
    cu = cu_dev([0, 30, T])

    def loss(xq):
        yq, _ = P.rope_qk_norm_fwd(xq, k, wq, wk, EPS, cu, 1e4, torch.empty_like(xq), torch.empty_like(k))
        return float((G.double() * yq.double()).sum())

    h = 1e-2
    fd = (loss(q + h * V) - loss(q - h * V)) / (2 * h)
    dq, _, _, _ = P.rope_qk_norm_bwd(G.clone(), torch.zeros_like(k), q, k, wq, wk, EPS, cu, 1e4)
    an = float((dq.double() * V.double()).sum())
    assert abs(fd - an) <= 1e-3 * (abs(an) + 1.0), (fd, an)


def norm_full_size(cfg, seeds):
    """One model-shaped batch at full size: the forward out of place and the
    backward in place, every element of every output against the oracle (bit
    for bit), and the weight gradients against the oracle's float64 sums over
    every token."""
    w = W.make_workload(cfg)
    T, D = w.T, w.D
    t = W.make_tensors(w, ("q", "k", "dq", "dk"), device=DEV)
    wq, wk = weights(D, seeds[0]), weights(D, seeds[1])
    cu = cu_dev(w.cu_seqlens)
    pos = oracle.segment_positions(w.cu_seqlens, T)
    assert (pos >= 0).all()  # every token of these batches is inside a sequence
    qo, ko = torch.empty_like(t["q"]), torch.empty_like(t["k"])
    P.rope_qk_norm_fwd(t["q"], t["k"], wq, wk, EPS, cu, w.theta, qo, ko)
    torch.cuda.synchronize()
    for x, y, wt, nm in ((t["q"], qo, wq, "q"), (t["k"], ko, wk, "k")):
        wv = w64(wt)

        def fwd_ref(s, e, xs, wv=wv):
            n, _ = oracle.rms_norm(xs, wv, EPS)
            return oracle.rotate(n, pos[s:e], w.theta, 1), None

        st, _ = check_chunks(y, [x], fwd_ref, f"{w.name} fwd {nm}")
        print("fwd", nm, st, flush=True)
        assert st["exact_fraction"] >= MIN_EXACT_FRACTION_AT_SCALE, st
    del qo, ko
    g = {nm: t["d" + nm].clone() for nm in ("q", "k")}  # the incoming gradients (dq, dk are overwritten)
    dq, dk, dwq, dwk = P.rope_qk_norm_bwd(t["dq"], t["dk"], t["q"], t["k"], wq, wk, EPS, cu, w.theta)
    torch.cuda.synchronize()
    for x, dx, dw, wt, nm in ((t["q"], dq, dwq, wq, "q"), (t["k"], dk, dwk, wk, "k")):
        wv = w64(wt)

        def bwd_ref(s, e, gs, xs, wv=wv):
            dn = oracle.rotate(gs, pos[s:e], w.theta, -1)
            dxr, dwc = oracle.rms_norm_bwd(dn, xs, wv, EPS)
            _, r = oracle.rms_norm(xs, wv, EPS)
            return dxr, (dwc, np.sum(np.abs(dn * xs * r[..., None]), axis=(0, 1)))

        st, aux = check_chunks(dx, [g[nm], x], bwd_ref, f"{w.name} bwd d{nm}")
        print("bwd", nm, st, flush=True)
        assert st["exact_fraction"] >= MIN_EXACT_FRACTION_AT_SCALE, st
        ref = np.sum([a[0] for a in aux], axis=0)
        S = np.sum([a[1] for a in aux], axis=0)
        check_dw(dw, ref, S, f"dw{nm} over every token")
    del t, g, dq, dk
    torch.cuda.empty_cache()


def test_norm_qwen3_8b_shape_full_size():
    """Qwen3-8B-shaped packed batch (T = 65536, 32 + 8 heads, D = 128, bf16):
    every element of the forward and backward outputs, and the weight
    gradients over every token."""
    norm_full_size(3, (31, 32))


def test_norm_long_context_full_size():
    """The 524,288-token single sequence (32 + 8 heads, D = 128, bf16; q has
    2^31 elements, so row offsets pass 2^32 bytes): every element of the
    forward and backward outputs, and the weight gradients over every token."""
    w = W.make_workload(5)
    assert w.T * w.Hq * w.D == 2 ** 31
    norm_full_size(5, (61, 62))
