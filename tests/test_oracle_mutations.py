"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each.

Every mutant is the oracle with one function swapped for a wrong variant; the
test passes when at least one pin in ``oracle_pins.ALL_PINS`` fails on it.
This shows the pins constrain every part of the computation: positions,
frequencies, angles, the sign convention, the pairing and each term.
"""

import numpy as np
import pytest

from oracle import rope_oracle as R
from tests import oracle_pins

_orig_rotate = R.rotate
_orig_cos_sin = R.cos_sin
_orig_inv_freq = R.inv_freq
_orig_positions = R.segment_positions
_orig_rope = R.rope
_orig_rotate_interleaved = R.rotate_interleaved
_orig_llama3 = R.llama3_inv_freq


def _rotate_with(fn):
    """Build a rotate() whose pair arithmetic is replaced by fn(x1, x2, c, s) -> (y1, y2)."""

    def rotate(x, pos, theta, direction):
        x = np.asarray(x, dtype=np.float64)
        N, H, D = x.shape
        c, s = R.cos_sin(np.asarray(pos), theta, D, direction)
        c, s = c[:, None, :], s[:, None, :]
        h = D // 2
        y = np.empty_like(x)
        y[:, :, :h], y[:, :, h:] = fn(x[:, :, :h], x[:, :, h:], c, s)
        return y

    return rotate


def _interleaved_rotate(x, pos, theta, direction):
    x = np.asarray(x, dtype=np.float64)
    N, H, D = x.shape
    c, s = R.cos_sin(np.asarray(pos), theta, D, direction)
    c, s = c[:, None, :], s[:, None, :]
    y = np.empty_like(x)
    y[:, :, 0::2] = x[:, :, 0::2] * c - x[:, :, 1::2] * s
    y[:, :, 1::2] = x[:, :, 1::2] * c + x[:, :, 0::2] * s
    return y


def _offset_last(cu, T, off):
    pos = _orig_positions(cu, T)
    c = np.asarray(cu, dtype=np.int64)
    if c.size > 1:
        pos[int(c[-2]):int(c[-1])] += off
    return pos


def _half_with_freq(x, pos, freq, direction):
    x = np.asarray(x, dtype=np.float64)
    r = x.shape[2]
    c, s = R.cos_sin_freq(pos, freq, direction)
    c, s = c[:, None, :], s[:, None, :]
    y = np.empty_like(x)
    y[:, :, : r // 2] = x[:, :, : r // 2] * c - x[:, :, r // 2:] * s
    y[:, :, r // 2:] = x[:, :, r // 2:] * c + x[:, :, : r // 2] * s
    return y


def _llama3_variant(theta, D, factor, low_freq_factor, high_freq_factor, original_max_position,
                    two_pi=2.0 * np.pi, swap_blend=False, swap_bands=False):
    base = R.inv_freq(theta, D)
    out = np.empty_like(base)
    L = original_max_position
    for i, f in enumerate(base):
        w = two_pi / f
        low, high = w > L / low_freq_factor, w < L / high_freq_factor
        if swap_bands:
            low, high = high, low
        if high:
            out[i] = f
        elif low:
            out[i] = f / factor
        else:
            s = (L / w - low_freq_factor) / (high_freq_factor - low_freq_factor)
            out[i] = (1.0 - s) * f + s * f / factor if swap_blend else (1.0 - s) * f / factor + s * f
    return out


def _rope_partial_full_freqs(x, cu, theta, direction, *, pos_offset=0, rotary_dim=None, pairing="half", scaling=None):
    x = np.asarray(x, dtype=np.float64)
    T, H, D = x.shape
    r = D if rotary_dim in (None, 0) else int(rotary_dim)
    pos = R.segment_positions(cu, T, pos_offset)
    y = x.copy()
    inside = pos >= 0
    f = R.inv_freq(theta, D)[: r // 2]  # the full head's frequencies
    xi = x[inside][:, :, :r]
    if pairing == "interleaved":
        y[inside, :, :r] = R.rotate_interleaved(xi, pos[inside], f, direction)
    else:
        y[inside, :, :r] = _half_with_freq(xi, pos[inside], f, direction)
    return y


MUTANTS = {
    # sign and direction conventions
    "sin_sign_flipped": ("cos_sin", lambda pos, th, D, d: (lambda c, s: (c, -s))(*_orig_cos_sin(pos, th, D, d))),
    "direction_ignored": ("cos_sin", lambda pos, th, D, d: _orig_cos_sin(pos, th, D, 1)),
    "cos_sin_swapped": ("cos_sin", lambda pos, th, D, d: (lambda c, s: (s, c))(*_orig_cos_sin(pos, th, D, d))),
    "angle_in_float32": (
        "cos_sin",
        lambda pos, th, D, d: (
            lambda a: (np.cos(a), d * np.sin(a))
        )((np.asarray(pos, np.float64)[:, None] * _orig_inv_freq(th, D)[None, :]).astype(np.float32).astype(np.float64)),
    ),
    # frequencies
    "freq_exponent_i_over_D": ("inv_freq", lambda th, D: np.power(float(th), -np.arange(D // 2) / float(D))),
    "freq_index_shifted": ("inv_freq", lambda th, D: np.power(float(th), -(2.0 * (np.arange(D // 2) + 1)) / D)),
    "freq_in_float32": ("inv_freq", lambda th, D: _orig_inv_freq(th, D).astype(np.float32).astype(np.float64)),
    # positions
    "no_restart_at_boundaries": (
        "segment_positions",
        lambda cu, T, off=0: np.where(_orig_positions(cu, T, off) >= 0, np.arange(T) - int(np.asarray(cu)[0]), -1),
    ),
    "positions_start_at_one": (
        "segment_positions",
        lambda cu, T, off=0: np.where(_orig_positions(cu, T, off) >= 0, _orig_positions(cu, T, off) + 1, -1),
    ),
    "outside_tokens_rotated": (
        "segment_positions",
        lambda cu, T, off=0: np.where(_orig_positions(cu, T, off) >= 0, _orig_positions(cu, T, off), np.arange(T)),
    ),
    # the position offset of a shard
    "pos_offset_ignored": ("segment_positions", lambda cu, T, off=0: _orig_positions(cu, T)),
    "pos_offset_on_every_segment": (
        "segment_positions",
        lambda cu, T, off=0: np.where(_orig_positions(cu, T) >= 0, _orig_positions(cu, T) + off, -1),
    ),
    "pos_offset_on_last_segment": ("segment_positions", lambda cu, T, off=0: _offset_last(cu, T, off)),
    # the pair arithmetic
    "dropped_cross_term": ("rotate", _rotate_with(lambda x1, x2, c, s: (x1 * c, x2 * c + x1 * s))),
    "one_sided_sign": ("rotate", _rotate_with(lambda x1, x2, c, s: (x1 * c - x2 * s, x2 * c - x1 * s))),
    "halves_swapped": ("rotate", _rotate_with(lambda x1, x2, c, s: (x2 * c + x1 * s, x1 * c - x2 * s))),
    "transposed_rotation": ("rotate", _rotate_with(lambda x1, x2, c, s: (x1 * c + x2 * s, x2 * c - x1 * s))),
    "interleaved_pairing": ("rotate", _interleaved_rotate),
    # interleaved pairing
    "interleaved_as_rotate_half": ("rotate_interleaved", lambda x, pos, f, d: _half_with_freq(x, pos, f, d)),
    "interleaved_transposed": (
        "rotate_interleaved",
        lambda x, pos, f, d: _orig_rotate_interleaved(x, pos, f, -d),
    ),
    # llama3 frequency rescaling
    "llama3_wavelength_without_2pi": ("llama3_inv_freq", lambda th, D, **kw: _llama3_variant(th, D, two_pi=1.0, **kw)),
    "llama3_blend_swapped": ("llama3_inv_freq", lambda th, D, **kw: _llama3_variant(th, D, swap_blend=True, **kw)),
    "llama3_bands_swapped": ("llama3_inv_freq", lambda th, D, **kw: _llama3_variant(th, D, swap_bands=True, **kw)),
    # partial rotary dim
    "partial_uses_full_head_freqs": ("rope", lambda *a, **kw: _rope_partial_full_freqs(*a, **kw)),
    "partial_rotates_whole_head": ("rope", lambda x, cu, th, d, **kw: _orig_rope(x, cu, th, d, **{**kw, "rotary_dim": None})),
    # float32-convention angles
    "fp32_mode_ignored": ("fp32_angles", lambda pos, f: np.asarray(pos, np.float64)[:, None] * np.asarray(f)[None, :]),
    "fp32_only_frequencies_rounded": (
        "fp32_angles",
        lambda pos, f: np.asarray(pos, np.float64)[:, None] * np.asarray(f).astype(np.float32).astype(np.float64)[None, :],
    ),
    "fp32_only_product_rounded": (
        "fp32_angles",
        lambda pos, f: (np.asarray(pos, np.float64)[:, None] * np.asarray(f)[None, :]).astype(np.float32).astype(np.float64),
    ),
    "fp32_position_not_rounded": (
        "fp32_angles",
        lambda pos, f: (np.asarray(pos, np.float64)[:, None] * np.asarray(f).astype(np.float32).astype(np.float64)[None, :])
        .astype(np.float32).astype(np.float64),
    ),
    # the fused call
    "k_left_unrotated": ("rope_qk", lambda q, k, cu, th, d: (_orig_rope(q, cu, th, d), np.asarray(k, np.float64).copy())),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(R, attr, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(R)
        except Exception:  # any failure of a pin is a detection
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"


# ---------------------------------------------------------------------------
# the fp16 rounding helper
# ---------------------------------------------------------------------------

_orig_fp16 = R.fp16_rne


def _fp16_variant(y, bits=11, sub_exp=24, rnd=np.rint, overflow=True):
    y = np.asarray(y, dtype=np.float64)
    m, e = np.frexp(y)
    r = np.ldexp(rnd(m * 2.0 ** bits), e - bits)
    small = np.abs(y) < 2.0 ** -14
    r = np.where(small, np.ldexp(rnd(np.ldexp(y, sub_exp)), -sub_exp), r)
    if overflow:
        r = np.where(np.abs(r) > 65504.0, np.copysign(np.inf, y), r)
    return r


FP16_MUTANTS = {
    "truncates": lambda y: _fp16_variant(y, rnd=np.trunc),
    "ties_away_from_zero": lambda y: _fp16_variant(y, rnd=lambda v: np.sign(v) * np.floor(np.abs(v) + 0.5)),
    "ten_significant_bits": lambda y: _fp16_variant(y, bits=10),
    "subnormal_grid_2^-25": lambda y: _fp16_variant(y, sub_exp=25),
    "no_overflow_to_inf": lambda y: _fp16_variant(y, overflow=False),
}


@pytest.mark.parametrize("name", sorted(FP16_MUTANTS))
def test_fp16_pins_catch_mutant(name, monkeypatch):
    from tests import test_oracle

    import oracle

    monkeypatch.setattr(R, "fp16_rne", FP16_MUTANTS[name])
    monkeypatch.setattr(oracle, "fp16_rne", FP16_MUTANTS[name])  # the package re-exports the module's names
    with pytest.raises(AssertionError):
        test_oracle.test_fp16_rne_hand_cases()
