"""fp64 CPU oracle for the fused QK rotary position embedding over packed
variable-length batches.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path (the HIP library and its Python binding) never imports, calls or links it,
and it shares no code, tables or constants with that path.

What is computed, and where it comes from
-----------------------------------------
The pages never print the rotary formula; they describe its properties:
q and k are rotated by one fused in-place kernel that handles variable-length
(packed) input ("Unsloth prétend accélérer 5 fois l'entraînement des LLM avec
de nouveaux noyaux Triton et un auto-packing", seventnews.com, the paragraph
on the fused QK RoPE kernel), packed sequences keep their length metadata so
nothing leaks between samples and packed losses equal unpacked ones (same
article, auto-packing paragraph), and Chronicals fuses "QK-RoPE" in its
kernels ("Chronicals: A High-Performance Framework for LLM Fine-Tuning with
3.51x Speedup over Unsloth", abstract, optimisation (1)).

The plainest reading consistent with that is the standard rotary position
embedding of RoFormer (Su et al., 2021: the block-diagonal rotary matrix of
its general form, realised element-wise), in the "rotate_half" layout that
pairs element i with element i + D/2 of each head:

    inv_freq[i] = theta ** (-(2 i) / D)                 i = 0 .. D/2-1
    angle[t, i] = pos[t] * inv_freq[i]
    y[t,h,i]       = x[t,h,i]       cos(angle) - x[t,h,i+D/2] sin(angle)
    y[t,h,i+D/2]   = x[t,h,i+D/2]   cos(angle) + x[t,h,i]     sin(angle)

pos[t] restarts at 0 at every packed-sequence boundary.  The backward pass is
the transpose of that orthogonal map, i.e. the same rotation by -angle applied
to the incoming gradients.

Everything is numpy float64, one operation at a time, no blocking or fusion.
Reduced-precision outputs are produced by exact round-to-nearest-even of the
float64 result (``bf16_rne``), a single rounding.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "segment_positions",
    "inv_freq",
    "cos_sin",
    "rotate",
    "rope",
    "rope_qk",
    "bf16_rne",
    "bf16_bits",
    "bits_to_f64",
    "ulp_distance_bf16",
]


def _check_cu(cu_seqlens, T: int) -> np.ndarray:
    cu = np.asarray(cu_seqlens, dtype=np.int64).ravel()
    if cu.size < 1:
        raise ValueError("cu_seqlens needs at least one entry")
    if cu[0] < 0 or np.any(np.diff(cu) < 0) or cu[-1] > T:
        raise ValueError("cu_seqlens must be non-decreasing within [0, T]")
    return cu


def segment_positions(cu_seqlens, T: int) -> np.ndarray:
    """Position of each of the T tokens inside its own packed sequence.

    Follows the auto-packing paragraph of the Unsloth article on
    seventnews.com: sequences are concatenated along one token axis and their
    length metadata is what keeps samples apart, so the position counter
    restarts at 0 at every boundary cu[s].  Tokens before cu[0] or from
    cu[nseq] on belong to no sequence and get -1 (they are left untouched).

    Built by repeating each segment's start offset over its length (no
    search), so it is a different construction from a binary search.
    """
    cu = _check_cu(cu_seqlens, T)
    pos = np.full(T, -1, dtype=np.int64)
    lengths = np.diff(cu)
    starts = cu[:-1]
    first, last = int(cu[0]), int(cu[-1])
    token = np.arange(first, last, dtype=np.int64)
    pos[first:last] = token - np.repeat(starts, lengths)
    return pos


def inv_freq(theta: float, D: int) -> np.ndarray:
    """Rotary frequencies theta^(-2i/D) for i < D/2, in float64.

    The base theta per workload is given by the shapes the pages' models use;
    the exponent follows RoFormer's frequency set.  Computed with float64
    ``pow`` (not rounded through float32).
    """
    if D < 2 or D % 2:
        raise ValueError("D must be even and >= 2")
    if not (np.isfinite(theta) and theta > 0):
        raise ValueError("theta must be finite and positive")
    i = np.arange(D // 2, dtype=np.float64)
    return np.power(np.float64(theta), -(2.0 * i) / np.float64(D))


def cos_sin(pos: np.ndarray, theta: float, D: int, direction: int):
    """cos and (direction * sin) of pos * inv_freq, float64 [N, D/2].

    direction = +1 for the forward pass, -1 for the backward pass (rotation
    by the negated angle, the transpose of the forward rotation).
    """
    if direction not in (1, -1):
        raise ValueError("direction must be +1 or -1")
    f = inv_freq(theta, D)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * f[None, :]
    return np.cos(ang), direction * np.sin(ang)


def rotate(x: np.ndarray, pos: np.ndarray, theta: float, direction: int) -> np.ndarray:
    """Rotate rows x[N, H, D] whose tokens sit at positions pos[N] (all >= 0).

    rotate_half pairing: element i of a head pairs with element i + D/2.
    Returns a new float64 array; x itself is not modified.
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 3:
        raise ValueError("x must be [N, H, D]")
    N, H, D = x.shape
    pos = np.asarray(pos, dtype=np.int64)
    if pos.shape != (N,) or np.any(pos < 0):
        raise ValueError("pos must be [N] and non-negative")
    c, s = cos_sin(pos, theta, D, direction)
    c = c[:, None, :]
    s = s[:, None, :]
    half = D // 2
    x1 = x[:, :, :half]
    x2 = x[:, :, half:]
    y = np.empty_like(x)
    y[:, :, :half] = x1 * c - x2 * s
    y[:, :, half:] = x2 * c + x1 * s
    return y


def rope(x: np.ndarray, cu_seqlens, theta: float, direction: int) -> np.ndarray:
    """Rotary embedding of a packed batch x[T, H, D] (float64 result).

    Tokens outside [cu[0], cu[nseq]) are returned unchanged.
    """
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    pos = segment_positions(cu_seqlens, T)
    y = x.copy()
    inside = pos >= 0
    if inside.any():
        y[inside] = rotate(x[inside], pos[inside], theta, direction)
    return y


def rope_qk(q: np.ndarray, k: np.ndarray, cu_seqlens, theta: float, direction: int):
    """Both tensors of the fused call: the same positions and angles for q and k."""
    return rope(q, cu_seqlens, theta, direction), rope(k, cu_seqlens, theta, direction)


# ---------------------------------------------------------------------------
# bf16 rounding and comparison helpers
# ---------------------------------------------------------------------------

_BF16_MIN_NORMAL = 2.0 ** -126
_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_rne(y: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    Normal range: write y = m * 2^e with 0.5 <= |m| < 1 (frexp); bfloat16
    keeps 8 significant bits, so the result is rint(m * 256) * 2^(e-8) with
    numpy's rint (round half to even).  Below the smallest normal the grid is
    fixed at 2^-133.  Overflow goes to +-inf, NaN stays NaN.  Returned as
    float64 holding exactly representable bfloat16 values.
    """
    y = np.asarray(y, dtype=np.float64)
    m, e = np.frexp(y)
    r = np.ldexp(np.rint(m * 256.0), e - 8)
    small = np.abs(y) < _BF16_MIN_NORMAL
    if np.any(small):
        r = np.where(small, np.ldexp(np.rint(np.ldexp(y, 133)), -133), r)
    # the largest finite bfloat16 is (2 - 2^-7) 2^127; anything that rounds past it is inf
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, y), r)
    return np.where(np.isnan(y), np.nan, r)


def bf16_bits(y: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float64 values that are exactly bfloat16-representable."""
    f = np.asarray(y, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """float64 values of uint16 bfloat16 bit patterns."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def _order_key(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_distance_bf16(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Number of bfloat16 grid steps between two bit patterns (+0 and -0 coincide)."""
    return np.abs(_order_key(a_bits) - _order_key(b_bits))
