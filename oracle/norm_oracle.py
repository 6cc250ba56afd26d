"""fp64 CPU oracle for per-head RMSNorm of q and k followed by the rotary
embedding, forward and backward.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it, and it shares nothing with the HIP path.

What is computed, and where it comes from
-----------------------------------------
"Chronicals: A High-Performance Framework for LLM Fine-Tuning with 3.51x
Speedup over Unsloth", abstract, optimisation (1): the fused kernels include
RMSNorm and QK-RoPE.  The pages print no formula for either.  The reading
implemented is RMSNorm as defined by Zhang and Sennrich ("Root Mean Square
Layer Normalization", 2019) applied to each head of q and of k on its own,
with one weight vector of length D per tensor shared by all of its heads,
and then the rotary embedding of ``rope_oracle.rope`` (same positions,
frequencies and options):

    m      = (1/D) sum_j x_j^2            over the D elements of one head
    r      = 1 / sqrt(m + eps)
    n_j    = x_j * r * w_j
    y      = rope(n)                       (rotation by +angle)

Tokens outside [cu[0], cu[nseq]) are neither normalised nor rotated, as the
rotation alone leaves them.  Per-head placement of the norm before the
rotation is the Qwen3 architecture's (a model the pages name); it is not on
the pages themselves.

Backward, for a loss L with dL/dy = dy: the rotation is orthogonal, so
dL/dn = rope(dy, direction=-1).  With g_j = (dL/dn_j) w_j, the chain rule
through r = (m + eps)^(-1/2), dr/dx_k = -r^3 x_k / D, gives

    dL/dx_k = r * (g_k - x_k * r^2 * (sum_j g_j x_j) / D)
    dL/dw_j = sum over every normalised head of (dL/dn_j) * x_j * r

Everything is numpy float64, one step at a time.
"""

from __future__ import annotations

import numpy as np

from .rope_oracle import rope, segment_positions

__all__ = ["rms_norm", "rms_norm_bwd", "norm_rope", "norm_rope_bwd"]


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float):
    """RMSNorm over the last axis: returns (x * r * w, r) in float64, r with the last axis dropped."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if w.shape != x.shape[-1:]:
        raise ValueError("w must have one entry per element of the last axis")
    if not (eps > 0 and np.isfinite(eps)):
        raise ValueError("eps must be finite and > 0")
    m = np.mean(x * x, axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(m + eps)
    return x * r * w, r[..., 0]


def rms_norm_bwd(dn: np.ndarray, x: np.ndarray, w: np.ndarray, eps: float):
    """Gradients of sum(dn * rms_norm(x, w, eps)[0]) with respect to x (same
    shape as x) and to w (summed over every leading index)."""
    x = np.asarray(x, dtype=np.float64)
    dn = np.asarray(dn, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    D = x.shape[-1]
    _, r = rms_norm(x, w, eps)
    r = r[..., None]
    g = dn * w
    proj = np.sum(g * x, axis=-1, keepdims=True) / D
    dx = r * (g - x * r * r * proj)
    dw = np.sum((dn * x * r).reshape(-1, D), axis=0)
    return dx, dw


def norm_rope(x: np.ndarray, w: np.ndarray, eps: float, cu_seqlens, theta: float, **variant):
    """Forward of one tensor x[T, H, D]: (y, rstd) with y float64 [T, H, D]
    and rstd float64 [T, H] (NaN for tokens outside every sequence).
    ``variant`` takes the keyword options of ``rope``."""
    x = np.asarray(x, dtype=np.float64)
    T, H, D = x.shape
    inside = segment_positions(cu_seqlens, T, variant.get("pos_offset", 0)) >= 0
    n, r = rms_norm(x, w, eps)
    y = rope(n, cu_seqlens, theta, 1, **variant)
    y[~inside] = x[~inside]
    r[~inside] = np.nan
    return y, r


def norm_rope_bwd(dy: np.ndarray, x: np.ndarray, w: np.ndarray, eps: float, cu_seqlens, theta: float, **variant):
    """Backward of ``norm_rope`` for one tensor: (dx [T, H, D], dw [D]).

    Tokens outside every sequence pass dy through unchanged (the forward is
    the identity there) and add nothing to dw."""
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    T, H, D = x.shape
    inside = segment_positions(cu_seqlens, T, variant.get("pos_offset", 0)) >= 0
    dn = rope(dy, cu_seqlens, theta, -1, **variant)
    dx = dy.copy()
    dw = np.zeros(D)
    if inside.any():
        dxi, dw = rms_norm_bwd(dn[inside], x[inside], w, eps)
        dx[inside] = dxi
    return dx, dw
