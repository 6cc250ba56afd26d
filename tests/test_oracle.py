"""The fp64 oracle against its pins (CPU only)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import rope_oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(rope_oracle)


def test_brute_positions_helper():
    # the brute-force counter itself on a hand-checked case
    assert oracle_pins.brute_positions([0, 2, 2, 5], 6) == [0, 1, 0, 1, 2, -1]


def test_rejects_bad_metadata():
    with pytest.raises(ValueError):
        oracle.segment_positions(np.array([0, 5, 3]), 8)
    with pytest.raises(ValueError):
        oracle.segment_positions(np.array([0, 9]), 8)
    with pytest.raises(ValueError):
        oracle.inv_freq(0.0, 64)
    with pytest.raises(ValueError):
        oracle.inv_freq(1e4, 7)


# ---------------------------------------------------------------------------
# bf16 rounding used for the reference outputs
# ---------------------------------------------------------------------------

def _bf16(v):
    return float(oracle.bf16_rne(np.array([v]))[0])


def test_bf16_rne_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert _bf16(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert _bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    # one float64 ulp either side of a tie decides it
    assert _bf16(1.0 + 2.0 ** -8 + 2.0 ** -52) == 1.0 + 2.0 ** -7
    assert _bf16(1.0 + 2.0 ** -8 - 2.0 ** -52) == 1.0
    assert _bf16(-(1.0 + 2.0 ** -8 + 2.0 ** -52)) == -(1.0 + 2.0 ** -7)
    # exactly representable values are kept; signed zero is kept
    for v in (0.5, -3.0, 1.0 + 2.0 ** -7, 2.0 ** -126, 2.0 ** -133):
        assert _bf16(v) == v
    assert np.signbit(oracle.bf16_rne(np.array([-0.0]))[0])


def test_bf16_rne_subnormal_and_overflow():
    assert _bf16(2.0 ** -134) == 0.0  # tie between 0 and 2^-133 goes to 0 (even)
    assert _bf16(3 * 2.0 ** -134) == 2.0 ** -132  # tie between 2^-133 and 2^-132 goes to even 2*2^-133
    assert _bf16(2.0 ** -126 - 2.0 ** -140) == 2.0 ** -126
    assert _bf16(3.5e38) == np.inf and _bf16(-3.5e38) == -np.inf
    assert _bf16(3.3e38) == float(torch.tensor(3.3e38, dtype=torch.float32).to(torch.bfloat16))
    assert np.isnan(_bf16(np.nan))


def test_bf16_rne_matches_torch_on_fp32_values():
    """On float32-representable inputs, torch's float32->bfloat16 cast (RNE) is a second implementation."""
    rng = np.random.default_rng(5)
    f = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-36).astype(np.float32),
        # exact ties: low 16 bits = 0x8000
        ((rng.integers(0x3F000000, 0x40800000, 20000, dtype=np.uint32) & 0xFFFF0000) | 0x8000).view(np.float32),
    ])
    ours = oracle.bf16_bits(oracle.bf16_rne(f.astype(np.float64)))
    theirs = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_ulp_distance():
    a = np.array([0x3F80, 0x3F80, 0x0000, 0x8000, 0x0001, 0xBF80], dtype=np.uint16)
    b = np.array([0x3F80, 0x3F81, 0x8000, 0x8001, 0x8001, 0xBF82], dtype=np.uint16)
    assert list(oracle.ulp_distance_bf16(a, b)) == [0, 1, 0, 1, 2, 2]
    v = np.array([1.0, -2.5, 0.15625])
    assert np.array_equal(oracle.bits_to_f64(oracle.bf16_bits(v)), v)


def test_fp16_rne_hand_cases():
    """Ties to even, subnormal grid and the overflow boundary, worked out by hand."""
    cases = [
        (1.0 + 2.0 ** -11, 1.0),                   # halfway between 1 and 1 + 2^-10: even is 1
        (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),   # halfway between 1 + 2^-10 and 1 + 2^-9: even is 1 + 2^-9
        (1.0 + 2.0 ** -11 + 2.0 ** -40, 1.0 + 2.0 ** -10),  # just above the tie
        (-(1.0 + 2.0 ** -11), -1.0),
        (65504.0, 65504.0),
        (65519.99, 65504.0),                       # below the midpoint 65520
        (65520.0, float("inf")),                   # the midpoint rounds to even, past the largest finite
        (2.0 ** -14, 2.0 ** -14),                  # smallest normal
        (2.0 ** -25, 0.0),                         # halfway between 0 and 2^-24: even is 0
        (3 * 2.0 ** -25, 2.0 ** -23),              # halfway between 2^-24 and 2^-23: even is 2^-23
        (5 * 2.0 ** -26, 2.0 ** -24),              # 1.25 * 2^-24
        (2.0 ** -14 - 2.0 ** -25, 2.0 ** -14),     # tie at the top of the subnormal range: even is 2^-14
    ]
    for y, want in cases:
        got = float(oracle.fp16_rne(np.array([y]))[0])
        assert got == want, (y, got, want)
    assert np.isnan(oracle.fp16_rne(np.array([np.nan]))[0])


def test_fp16_rne_matches_an_independent_conversion():
    """numpy's float64 -> float16 cast is a separate implementation of the same rounding."""
    rng = np.random.default_rng(5)
    y = np.concatenate([rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 5, size=200000),
                        (np.arange(-4096, 4096) + 0.5) * 2.0 ** -24,  # every subnormal tie
                        1.0 + (np.arange(2048) + 0.5) * 2.0 ** -10])  # every tie in [1, 2)
    with np.errstate(over="ignore"):
        ref = y.astype(np.float16).astype(np.float64)
    got = oracle.fp16_rne(y)
    assert np.array_equal(got, ref)
    assert np.array_equal(oracle.fp16_bits_to_f64(oracle.fp16_bits(got)), got)
