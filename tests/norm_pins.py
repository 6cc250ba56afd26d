"""Pins that tie the RMSNorm + RoPE oracle (oracle/norm_oracle.py) to
mathematics rather than to itself.

Each ``pin_*`` takes the oracle module (or a copy with a planted mistake) and
raises AssertionError when it disagrees with:

* hand-worked values: a constant head (r = 1/sqrt(c^2 + eps)) and a D = 2
  head, where the rotation is the closed form (cos p, sin p) of the position;
* central finite differences of sum(G * y) in float64, for dx and dw, through
  positions, several sequences, grouped heads and tokens outside;
* invariants: unit mean square without eps, scale invariance and dx
  orthogonal to x when eps is negligible, per-head mean square kept by the
  rotation, tokens outside untouched.
"""

from __future__ import annotations

import math

import numpy as np


def _rng(seed):
    return np.random.default_rng(seed)


def pin_constant_head(N):
    """x = c on every element: m = c^2, r = 1/sqrt(c^2 + eps); c = 2, eps = 5 gives r = 1/3."""
    D = 16
    x = np.full((3, 2, D), 2.0)
    w = np.arange(1, D + 1, dtype=np.float64)
    n, r = N.rms_norm(x, w, 5.0)
    assert np.all(r == 1.0 / 3.0)
    assert np.allclose(n, 2.0 / 3.0 * w, rtol=2e-16, atol=0)


def pin_d2_closed_form(N):
    """D = 2, x = (3, 4), w = (1, 2), eps = 1/2: m = 12.5, r = 1/sqrt(13), the
    normalised head is (3, 8)/sqrt(13); D = 2 has the single frequency 1, so the
    token at position p rotates by p radians."""
    s13 = math.sqrt(13.0)
    n1, n2 = 3.0 / s13, 8.0 / s13
    ps = [0, 1, 5, 1000, 77777]
    T = len(ps)
    x = np.tile(np.array([3.0, 4.0]), (T, 1, 1))
    for t, p in enumerate(ps):
        cu = [t, t + 1]  # token t alone, at position pos_offset
        y, r = N.norm_rope(x, np.array([1.0, 2.0]), 0.5, cu, 1e4, pos_offset=p)
        assert abs(r[t, 0] - 1.0 / s13) <= 1e-16
        c, s = math.cos(p), math.sin(p)
        assert abs(y[t, 0, 0] - (n1 * c - n2 * s)) <= 1e-15, p
        assert abs(y[t, 0, 1] - (n2 * c + n1 * s)) <= 1e-15, p


def pin_unit_mean_square(N):
    """With eps negligible and w = 1 the normalised head has mean square 1,
    and scaling a head by any a > 0 does not change it."""
    rng = _rng(31)
    x = rng.standard_normal((50, 3, 64))
    n, _ = N.rms_norm(x, np.ones(64), 1e-300)
    assert np.allclose(np.mean(n * n, axis=-1), 1.0, rtol=1e-14, atol=0)
    n2, _ = N.rms_norm(x * 37.5, np.ones(64), 1e-300)
    assert np.allclose(n2, n, rtol=1e-14, atol=1e-15)


def pin_rotation_keeps_mean_square(N):
    """The rotation is orthogonal on every pair, so each head of y has the mean
    square of the normalised head: m / (m + eps) when w = 1."""
    rng = _rng(32)
    T, H, D = 40, 3, 32
    x = rng.standard_normal((T, H, D))
    eps = 0.3
    y, r = N.norm_rope(x, np.ones(D), eps, [0, 17, T], 1e4)
    m = np.mean(x * x, axis=-1)
    assert np.allclose(np.mean(y * y, axis=-1), m / (m + eps), rtol=1e-13, atol=0)
    assert np.allclose(r, 1.0 / np.sqrt(m + eps), rtol=1e-15, atol=0)


def pin_outside_untouched(N):
    rng = _rng(33)
    T, H, D = 12, 2, 8
    x = rng.standard_normal((T, H, D))
    dy = rng.standard_normal((T, H, D))
    w = rng.standard_normal(D)
    cu = [3, 5, 5, 8]
    y, r = N.norm_rope(x, w, 1e-6, cu, 1e4)
    assert np.array_equal(y[:3], x[:3]) and np.array_equal(y[8:], x[8:])
    assert np.all(np.isnan(r[:3])) and np.all(np.isfinite(r[3:8]))
    dx, dw = N.norm_rope_bwd(dy, x, w, 1e-6, cu, 1e4)
    assert np.array_equal(dx[:3], dy[:3]) and np.array_equal(dx[8:], dy[8:])
    dx_in, dw_in = N.norm_rope_bwd(dy[3:8], x[3:8], w, 1e-6, [0, 2, 2, 5], 1e4)
    assert np.array_equal(dw, dw_in)  # outside tokens add nothing to dw


def _fd_case(N, variant, seed):
    rng = _rng(seed)
    T, H, D = 6, 2, 8
    x = rng.standard_normal((T, H, D))
    w = rng.standard_normal(D)
    G = rng.standard_normal((T, H, D))
    cu = [1, 3, 6]  # token 0 outside; two sequences
    eps, theta = 0.05, 1e2

    def loss(xx, ww):
        return float(np.sum(G * N.norm_rope(xx, ww, eps, cu, theta, **variant)[0]))

    dx, dw = N.norm_rope_bwd(G, x, w, eps, cu, theta, **variant)
    h = 1e-6
    num_dx = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        num_dx[idx] = (loss(xp, w) - loss(xm, w)) / (2 * h)
    num_dw = np.zeros(D)
    for j in range(D):
        wp, wm = w.copy(), w.copy()
        wp[j] += h
        wm[j] -= h
        num_dw[j] = (loss(x, wp) - loss(x, wm)) / (2 * h)
    scale = 1.0 + np.max(np.abs(num_dx))
    assert np.max(np.abs(dx - num_dx)) <= 1e-7 * scale, (variant, np.max(np.abs(dx - num_dx)))
    assert np.max(np.abs(dw - num_dw)) <= 1e-7 * (1.0 + np.max(np.abs(num_dw))), (variant, dw - num_dw)


def pin_backward_finite_differences(N):
    """dx and dw against central differences of sum(G * y), loss evaluated by the
    forward alone; rotate_half and interleaved pairing, with a position offset."""
    _fd_case(N, {}, 34)
    _fd_case(N, dict(pairing="interleaved", pos_offset=1000), 35)


def pin_backward_orthogonal_to_input(N):
    """With eps negligible the forward is scale invariant per head, so the
    gradient is orthogonal to the input head: sum_k dx_k x_k = 0."""
    rng = _rng(36)
    T, H, D = 30, 4, 64
    x = rng.standard_normal((T, H, D))
    dy = rng.standard_normal((T, H, D))
    w = rng.standard_normal(D)
    dx, _ = N.norm_rope_bwd(dy, x, w, 1e-300, [0, 11, T], 1e6)
    dots = np.sum(dx * x, axis=-1)
    assert np.max(np.abs(dots)) <= 1e-12 * np.max(np.abs(dx)) * np.sqrt(D) * 8


ALL_NORM_PINS = [
    pin_constant_head,
    pin_d2_closed_form,
    pin_unit_mean_square,
    pin_rotation_keeps_mean_square,
    pin_outside_untouched,
    pin_backward_finite_differences,
    pin_backward_orthogonal_to_input,
]
