"""The RMSNorm + RoPE oracle against its pins (CPU), and planted mistakes that
the pins must catch."""

import numpy as np
import pytest

import oracle.norm_oracle as N
from tests import norm_pins


@pytest.mark.parametrize("pin", norm_pins.ALL_NORM_PINS, ids=lambda f: f.__name__)
def test_norm_pin(pin):
    pin(N)


_orig_rms_norm = N.rms_norm
_orig_rms_norm_bwd = N.rms_norm_bwd
_orig_rope = N.rope


def _rms_variant(x, w, eps, eps_outside=False, use_sum=False, no_weight=False):
    x = np.asarray(x, dtype=np.float64)
    m = np.sum(x * x, axis=-1, keepdims=True) if use_sum else np.mean(x * x, axis=-1, keepdims=True)
    r = 1.0 / (np.sqrt(m) + eps) if eps_outside else 1.0 / np.sqrt(m + eps)
    return (x * r if no_weight else x * r * np.asarray(w)), r[..., 0]


def _bwd_variant(dn, x, w, eps, proj_sign=-1.0, r_power=2, no_proj=False, dw_without_r=False):
    x = np.asarray(x, dtype=np.float64)
    dn = np.asarray(dn, dtype=np.float64)
    D = x.shape[-1]
    r = (1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps))
    g = dn * w
    proj = np.sum(g * x, axis=-1, keepdims=True) / D
    dx = r * g if no_proj else r * (g + proj_sign * x * r ** r_power * proj)
    dw = np.sum((dn * x * (1.0 if dw_without_r else r)).reshape(-1, D), axis=0)
    return dx, dw


def _rope_forward_in_bwd(x, cu, theta, direction, **kw):
    return _orig_rope(x, cu, theta, 1, **kw)


def _norm_after_rope(x, w, eps, cu, theta, **variant):
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    inside = N.segment_positions(cu, T, variant.get("pos_offset", 0)) >= 0
    y, r = _orig_rms_norm(_orig_rope(x, cu, theta, 1, **variant), w, eps)
    y[~inside] = x[~inside]
    r[~inside] = np.nan
    return y, r


NORM_MUTANTS = {
    "eps_outside_sqrt": ("rms_norm", lambda x, w, eps: _rms_variant(x, w, eps, eps_outside=True)),
    "sum_not_mean": ("rms_norm", lambda x, w, eps: _rms_variant(x, w, eps, use_sum=True)),
    "weight_ignored": ("rms_norm", lambda x, w, eps: _rms_variant(x, w, eps, no_weight=True)),
    "bwd_projection_dropped": ("rms_norm_bwd", lambda dn, x, w, eps: _bwd_variant(dn, x, w, eps, no_proj=True)),
    "bwd_projection_sign": ("rms_norm_bwd", lambda dn, x, w, eps: _bwd_variant(dn, x, w, eps, proj_sign=1.0)),
    "bwd_r_not_squared": ("rms_norm_bwd", lambda dn, x, w, eps: _bwd_variant(dn, x, w, eps, r_power=1)),
    "bwd_dw_without_r": ("rms_norm_bwd", lambda dn, x, w, eps: _bwd_variant(dn, x, w, eps, dw_without_r=True)),
    "bwd_rotation_not_undone": ("rope", _rope_forward_in_bwd),
    "norm_after_rope": ("norm_rope", _norm_after_rope),
}


@pytest.mark.parametrize("name", sorted(NORM_MUTANTS))
def test_norm_pins_catch_mutant(name, monkeypatch):
    attr, fn = NORM_MUTANTS[name]
    monkeypatch.setattr(N, attr, fn)
    caught = []
    for pin in norm_pins.ALL_NORM_PINS:
        try:
            pin(N)
        except Exception:  # any failure of a pin is a detection
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
