"""Helpers shared by the GPU parity tests: compare HIP results with the oracle."""

from __future__ import annotations

import numpy as np
import torch

import oracle

FP32_TOL = 1e-5  # max-abs against the float64 oracle
BF16_MAX_ULP = 1  # bf16 grid steps from the oracle's correctly rounded value
FP16_MAX_ULP = 1  # fp16 grid steps from the oracle's correctly rounded value


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
