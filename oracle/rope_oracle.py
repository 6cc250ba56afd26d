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

Variants (``rope`` keyword arguments; the defaults give the formula above):

* ``pos_offset``: added to the positions of the first packed segment, i.e.
  the global position of the first token of a shard that starts inside a
  sequence.  The pages' "positions restart per sequence" rule is kept for
  every later segment.  Not on the pages; the plainest reading of sharding
  one long sequence over tokens.
* ``rotary_dim`` r < D: only elements [0, r) of each head are rotated, with
  the frequencies of a head of size r; elements [r, D) are left as they are.
* ``pairing="interleaved"``: element 2i pairs with 2i + 1 -- RoFormer's
  block-diagonal matrix taken literally, with no reordering of the head.
* ``scaling``: the Llama 3.1 frequency rescaling (the pages name Llama 3.1
  among the supported models but do not give the rule; it is restated here
  from the model family's published definition): frequencies whose
  wavelength 2 pi / f is shorter than ``original_max_position /
  high_freq_factor`` are kept, those longer than ``original_max_position /
  low_freq_factor`` are divided by ``factor``, and those in between are
  blended linearly in ``original_max_position / wavelength``.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "segment_positions",
    "inv_freq",
    "llama3_inv_freq",
    "cos_sin",
    "rotate",
    "rotate_interleaved",
    "cos_sin_freq",
    "fp32_angles",
    "rope",
    "rope_qk",
    "bf16_rne",
    "bf16_bits",
    "bits_to_f64",
    "ulp_distance_bf16",
    "fp16_rne",
    "fp16_bits",
    "fp16_bits_to_f64",
    "ulp_distance_16",
]


def _check_cu(cu_seqlens, T: int) -> np.ndarray:
    cu = np.asarray(cu_seqlens, dtype=np.int64).ravel()
    if cu.size < 1:
        raise ValueError("cu_seqlens needs at least one entry")
    if cu[0] < 0 or np.any(np.diff(cu) < 0) or cu[-1] > T:
        raise ValueError("cu_seqlens must be non-decreasing within [0, T]")
    return cu


def segment_positions(cu_seqlens, T: int, pos_offset: int = 0) -> np.ndarray:
    """Position of each of the T tokens inside its own packed sequence.

    Follows the auto-packing paragraph of the Unsloth article on
    seventnews.com: sequences are concatenated along one token axis and their
    length metadata is what keeps samples apart, so the position counter
    restarts at 0 at every boundary cu[s].  Tokens before cu[0] or from
    cu[nseq] on belong to no sequence and get -1 (they are left untouched).

    Built by repeating each segment's start offset over its length (no
    search), so it is a different construction from a binary search.
    ``pos_offset`` is added to the positions of segment 0 only.
    """
    cu = _check_cu(cu_seqlens, T)
    if pos_offset < 0:
        raise ValueError("pos_offset must be >= 0")
    pos = np.full(T, -1, dtype=np.int64)
    lengths = np.diff(cu)
    starts = cu[:-1]
    first, last = int(cu[0]), int(cu[-1])
    token = np.arange(first, last, dtype=np.int64)
    pos[first:last] = token - np.repeat(starts, lengths)
    if cu.size > 1:
        pos[int(cu[0]):int(cu[1])] += pos_offset
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


def llama3_inv_freq(theta: float, D: int, factor: float, low_freq_factor: float, high_freq_factor: float,
                    original_max_position: float) -> np.ndarray:
    """Llama 3.1 rescaling of ``inv_freq(theta, D)``, one frequency at a time.

    With L = original_max_position, wavelength w = 2 pi / f:
    w < L / high_freq_factor: f is kept; w > L / low_freq_factor: f / factor;
    otherwise, with s = (L / w - low_freq_factor) / (high_freq_factor - low_freq_factor),
    (1 - s) f / factor + s f.
    """
    if not (factor > 0 and original_max_position > 0 and high_freq_factor > low_freq_factor > 0):
        raise ValueError("need factor > 0, original_max_position > 0, high_freq_factor > low_freq_factor > 0")
    base = inv_freq(theta, D)
    out = np.empty_like(base)
    low_wavelen = original_max_position / low_freq_factor
    high_wavelen = original_max_position / high_freq_factor
    for i, f in enumerate(base):
        w = 2.0 * np.pi / f
        if w < high_wavelen:
            out[i] = f
        elif w > low_wavelen:
            out[i] = f / factor
        else:
            s = (original_max_position / w - low_freq_factor) / (high_freq_factor - low_freq_factor)
            out[i] = (1.0 - s) * f / factor + s * f
    return out


def cos_sin(pos: np.ndarray, theta: float, D: int, direction: int):
    """cos and (direction * sin) of pos * inv_freq, float64 [N, D/2].

    direction = +1 for the forward pass, -1 for the backward pass (rotation
    by the negated angle, the transpose of the forward rotation).
    """
    if direction not in (1, -1):
        raise ValueError("direction must be +1 or -1")
    return cos_sin_freq(pos, inv_freq(theta, D), direction)


def fp32_angles(pos: np.ndarray, freq: np.ndarray) -> np.ndarray:
    """Angles as a float32 frequency table forms them, float64 [N, len(freq)].

    Each frequency is rounded to float32, each position converted to
    float32, and the angle is their float32 product; every step is one IEEE
    round-to-nearest-even.  (Compatibility reading: the common tables of
    models trained this way hold float32 frequencies and multiply in
    float32; the pages fix neither convention.)
    """
    f32 = np.asarray(freq, dtype=np.float64).astype(np.float32)
    p32 = np.asarray(pos, dtype=np.float64).astype(np.float32)
    return (p32[:, None] * f32[None, :]).astype(np.float64)


def cos_sin_freq(pos: np.ndarray, freq: np.ndarray, direction: int, freq_precision: str = "fp64"):
    """cos and (direction * sin) of pos * freq for given frequencies, float64 [N, len(freq)].

    freq_precision "fp64": the angle is the float64 product; "fp32": the
    angle of ``fp32_angles``.  cos and sin are float64 either way.
    """
    if direction not in (1, -1):
        raise ValueError("direction must be +1 or -1")
    if freq_precision == "fp64":
        ang = np.asarray(pos, dtype=np.float64)[:, None] * np.asarray(freq, dtype=np.float64)[None, :]
    elif freq_precision == "fp32":
        ang = fp32_angles(pos, freq)
    else:
        raise ValueError("freq_precision is 'fp64' or 'fp32'")
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


def rotate_interleaved(x: np.ndarray, pos: np.ndarray, freq: np.ndarray, direction: int,
                       freq_precision: str = "fp64") -> np.ndarray:
    """Rotate rows x[N, H, r] pairing element 2i with 2i + 1 (frequency freq[i])."""
    x = np.asarray(x, dtype=np.float64)
    N, H, r = x.shape
    c, s = cos_sin_freq(pos, freq, direction, freq_precision)
    c = c[:, None, :]
    s = s[:, None, :]
    x1 = x[:, :, 0::2]
    x2 = x[:, :, 1::2]
    y = np.empty_like(x)
    y[:, :, 0::2] = x1 * c - x2 * s
    y[:, :, 1::2] = x2 * c + x1 * s
    return y


def rope(x: np.ndarray, cu_seqlens, theta: float, direction: int, *, pos_offset: int = 0, rotary_dim=None,
         pairing: str = "half", scaling=None, freq_precision: str = "fp64") -> np.ndarray:
    """Rotary embedding of a packed batch x[T, H, D] (float64 result).

    Tokens outside [cu[0], cu[nseq]) are returned unchanged, and so are the
    elements [rotary_dim, D) of every head.  ``scaling`` is None or a dict
    with the keys of ``llama3_inv_freq``; ``freq_precision`` "fp32" forms the
    angles as ``fp32_angles`` does (after any scaling).
    """
    x = np.asarray(x, dtype=np.float64)
    T, H, D = x.shape
    r = D if rotary_dim in (None, 0) else int(rotary_dim)
    if r < 2 or r % 2 or r > D:
        raise ValueError("rotary_dim must be even, in [2, D]")
    if pairing not in ("half", "interleaved"):
        raise ValueError("pairing is 'half' or 'interleaved'")
    pos = segment_positions(cu_seqlens, T, pos_offset)
    y = x.copy()
    inside = pos >= 0
    if not inside.any():
        return y
    if pairing == "half" and scaling is None and freq_precision == "fp64":
        y[inside, :, :r] = rotate(x[inside][:, :, :r], pos[inside], theta, direction)
        return y
    freq = inv_freq(theta, r) if scaling is None else llama3_inv_freq(theta, r, **scaling)
    if pairing == "interleaved":
        y[inside, :, :r] = rotate_interleaved(x[inside][:, :, :r], pos[inside], freq, direction, freq_precision)
    else:
        c, s = cos_sin_freq(pos[inside], freq, direction, freq_precision)
        c, s = c[:, None, :], s[:, None, :]
        xi = x[inside]
        x1, x2 = xi[:, :, : r // 2], xi[:, :, r // 2: r]
        y[inside, :, : r // 2] = x1 * c - x2 * s
        y[inside, :, r // 2: r] = x2 * c + x1 * s
    return y


def rope_qk(q: np.ndarray, k: np.ndarray, cu_seqlens, theta: float, direction: int, **variant):
    """Both tensors of the fused call: the same positions and angles for q and k."""
    return rope(q, cu_seqlens, theta, direction, **variant), rope(k, cu_seqlens, theta, direction, **variant)


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


# ---------------------------------------------------------------------------
# IEEE binary16 (fp16) rounding and comparison helpers
# ---------------------------------------------------------------------------

_FP16_MIN_NORMAL = 2.0 ** -14
_FP16_MAX = (2.0 - 2.0 ** -10) * 2.0 ** 15  # 65504


def fp16_rne(y: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest IEEE half-precision value, ties to even.

    Normal range: y = m * 2^e with 0.5 <= |m| < 1 (frexp); half precision keeps
    11 significant bits, so the result is rint(m * 2^11) * 2^(e-11).  Below the
    smallest normal 2^-14 the grid is fixed at 2^-24.  Values that round past
    the largest finite half, 65504, become +-inf; NaN stays NaN.  Returned as
    float64 holding exactly representable half values.
    """
    y = np.asarray(y, dtype=np.float64)
    m, e = np.frexp(y)
    r = np.ldexp(np.rint(m * 2048.0), e - 11)
    small = np.abs(y) < _FP16_MIN_NORMAL
    if np.any(small):
        r = np.where(small, np.ldexp(np.rint(np.ldexp(y, 24)), -24), r)
    r = np.where(np.abs(r) > _FP16_MAX, np.copysign(np.inf, y), r)
    return np.where(np.isnan(y), np.nan, r)


def fp16_bits(y: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float64 values that are exactly half-representable."""
    return np.asarray(y, dtype=np.float64).astype(np.float16).view(np.uint16)


def fp16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """float64 values of uint16 half-precision bit patterns."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def ulp_distance_16(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Grid steps between two 16-bit sign-magnitude float patterns (bf16 or fp16; +0 and -0 coincide)."""
    return np.abs(_order_key(a_bits) - _order_key(b_bits))
