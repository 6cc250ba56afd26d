"""Helpers shared by the GPU parity tests: compare HIP results with the oracle."""

from __future__ import annotations

import numpy as np
import torch

import oracle

FP32_TOL = 1e-5  # max-abs against the float64 oracle
BF16_MAX_ULP = 1  # bf16 grid steps from the oracle's correctly rounded value
FP16_MAX_ULP = 1  # fp16 grid steps from the oracle's correctly rounded value
# Over billions of elements the kernels' float64 evaluation order (fused
# multiply-adds, the norm's weights folded into the table) and the oracle's
# (one operation at a time) can leave the two float64 values on either side
# of a rounding boundary of the 16-bit grid: a 1-ulp difference that the
# tolerance allows, seen once in 2^31 elements of the norm forward.  A
# double-rounding defect would show in about 2^-17 of all elements (ties of
# the float32 intermediate), so full-size checks also require at least this
# exact fraction.
MIN_EXACT_FRACTION_AT_SCALE = 1.0 - 2.0 ** -26


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a float32/bfloat16/float16 tensor on the host."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def check_against(gpu_out: torch.Tensor, ref: np.ndarray, what: str = "") -> dict:
    """Element-by-element check of a GPU output against the oracle's float64 values.

    fp32: max |gpu - ref| <= 1e-5.  bf16 / fp16: at most one grid step from
    the oracle's correctly rounded bf16 / fp16 (and we also count exact matches).
    """
    if gpu_out.dtype == torch.float32:
        err = np.abs(f64(gpu_out) - ref)
        m = float(err.max()) if err.size else 0.0
        assert m <= FP32_TOL, f"{what}: fp32 max-abs error {m}"
        return {"max_abs": m}
    if gpu_out.dtype == torch.float16:
        want, tol, name = oracle.fp16_bits(oracle.fp16_rne(ref)), FP16_MAX_ULP, "fp16"
    else:
        assert gpu_out.dtype == torch.bfloat16
        want, tol, name = oracle.bf16_bits(oracle.bf16_rne(ref)), BF16_MAX_ULP, "bf16"
    got = bits16(gpu_out)
    d = oracle.ulp_distance_16(got, want)
    m = int(d.max()) if d.size else 0
    exact = float(np.mean(d == 0)) if d.size else 1.0
    assert m <= tol, f"{what}: {name} max ulp {m} (exact fraction {exact})"
    return {"max_ulp": m, "exact_fraction": exact, "n": int(d.size)}


def sample_tokens(cu: np.ndarray, T: int, n_random: int, seed: int) -> np.ndarray:
    """First/last tokens, every segment's first and last token (up to 200 segments), and random ones."""
    rng = np.random.default_rng(seed)
    cu = np.asarray(cu, dtype=np.int64)
    idx = [0, T - 1]
    starts = cu[:-1][: 200]
    idx += list(starts) + list(np.maximum(cu[1:][: 200] - 1, 0))
    idx += list(rng.integers(0, T, size=n_random))
    idx = np.unique(np.clip(np.array(idx, dtype=np.int64), 0, T - 1))
    return idx


def check_chunks(out: torch.Tensor, inputs, ref_fn, what: str, chunk: int = 2048, threads: int = 16):
    """Every element of a GPU output [T, ...] (bf16/fp16) against the oracle, chunk by chunk.

    Token chunks of `out` and of the device tensors `inputs` are copied to
    the host one at a time and checked on a thread pool (numpy releases the
    GIL): ref_fn(s, e, *inputs_f64) returns (the oracle's float64 values of
    out[s:e], an auxiliary result or None); rounded once to the storage type
    they must lie within one ulp of the output.  Returns (stats, the
    auxiliary results in chunk order)."""
    import concurrent.futures as cf

    T = out.shape[0]
    fp16 = out.dtype == torch.float16
    rne, to_bits = (oracle.fp16_rne, oracle.fp16_bits) if fp16 else (oracle.bf16_rne, oracle.bf16_bits)

    def one(s, e, got, xs):
        ref, aux = ref_fn(s, e, *xs)
        want = to_bits(rne(ref))
        if np.array_equal(got, want):
            return got.size, got.size, 0, aux
        d = oracle.ulp_distance_16(got, want)
        return got.size, int((d == 0).sum()), int(d.max()), aux

    n = exact = worst = 0
    auxes = []
    pending = []

    def drain(f):
        nonlocal n, exact, worst
        a, b, c, aux = f.result()
        n, exact, worst = n + a, exact + b, max(worst, c)
        auxes.append(aux)

    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        for s in range(0, T, chunk):
            e = min(s + chunk, T)
            xs = [f64(x[s:e]) for x in inputs]
            pending.append(ex.submit(one, s, e, bits16(out[s:e]), xs))
            if len(pending) >= 2 * threads:  # bound the chunks held on the host
                drain(pending.pop(0))
        for f in pending:
            drain(f)
    stats = {"elements": n, "exact_fraction": exact / n if n else 1.0, "max_ulp": worst}
    assert n == out.numel(), (what, n)
    assert worst <= (FP16_MAX_ULP if fp16 else BF16_MAX_ULP), f"{what}: {stats}"
    return stats, auxes


def check_every_element(before: torch.Tensor, after: torch.Tensor, cu, theta: float, direction: int, what: str,
                        chunk: int = 2048, threads: int = 16) -> dict:
    """Every element of a rotated [T, H, D] bf16/fp16 tensor against the oracle.

    `before` holds the kernel's input, `after` its output (device tensors):
    the oracle's float64 rotation of the input, rounded once to the storage
    type, must lie within one ulp of the output, and tokens outside every
    sequence must be unchanged.  Returns the element count, the exact
    fraction and the largest ulp distance."""
    pos = oracle.segment_positions(cu, before.shape[0])

    def ref(s, e, x):
        p = pos[s:e]
        inside = p >= 0
        y = x.copy()
        if inside.any():
            y[inside] = oracle.rotate(x[inside], p[inside], theta, direction)
        return y, None

    stats, _ = check_chunks(after, [before], ref, what, chunk, threads)
    return stats
