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
        lambda cu, T: np.where(_orig_positions(cu, T) >= 0, np.arange(T) - int(np.asarray(cu)[0]), -1),
    ),
    "positions_start_at_one": ("segment_positions", lambda cu, T: np.where(_orig_positions(cu, T) >= 0, _orig_positions(cu, T) + 1, -1)),
    "outside_tokens_rotated": (
        "segment_positions",
        lambda cu, T: np.where(_orig_positions(cu, T) >= 0, _orig_positions(cu, T), np.arange(T)),
    ),
    # the pair arithmetic
    "dropped_cross_term": ("rotate", _rotate_with(lambda x1, x2, c, s: (x1 * c, x2 * c + x1 * s))),
    "one_sided_sign": ("rotate", _rotate_with(lambda x1, x2, c, s: (x1 * c - x2 * s, x2 * c - x1 * s))),
    "halves_swapped": ("rotate", _rotate_with(lambda x1, x2, c, s: (x2 * c + x1 * s, x1 * c - x2 * s))),
    "transposed_rotation": ("rotate", _rotate_with(lambda x1, x2, c, s: (x1 * c + x2 * s, x2 * c - x1 * s))),
    "interleaved_pairing": ("rotate", _interleaved_rotate),
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
