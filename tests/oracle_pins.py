"""Pins that tie the fp64 oracle to mathematics rather than to itself.

Each ``pin_*`` function takes the oracle module (or a copy with a planted
mistake) and raises AssertionError when it disagrees with an independent
statement of what RoPE computes:

* brute-force position counting over tiny packed batches;
* 50-digit mpmath values of the frequencies, cos and sin at the exact angle;
* the D = 2 closed form (the unit vectors rotate to (cos p, sin p) and
  (-sin p, cos p));
* RoFormer's block-diagonal rotary matrix, which pairs *adjacent* elements,
  written out entry by entry in mpmath and conjugated by the permutation that
  maps the rotate_half layout (i, i + D/2) onto adjacent pairs;
* complex multiplication (x_i + j x_{i+D/2}) * exp(j * direction * angle);
* invariants: identity at position 0, per-pair norm, backward after forward,
  dependence of q.k on the position difference only, packed = unpacked.

The pages print no formula and no worked numbers, so every value here comes
from mathematics; see the module docstring of the oracle for the reading.
"""

from __future__ import annotations

import math

import mpmath
import numpy as np

mpmath.mp.dps = 50

F64_EPS = 2.0 ** -52


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# positions
# ---------------------------------------------------------------------------

POSITION_CASES = [
    ([0, 7, 40, 104, 256], 256),
    ([0, 1, 2, 3], 5),  # length-1 sequences, two trailing tokens outside
    ([0, 0, 0, 4, 4, 9], 9),  # empty segments
    ([3, 5, 5, 8], 12),  # tokens before cu[0] and after cu[nseq]
    ([0], 4),  # nseq = 0: nothing is inside
    ([0, 16], 16),
]


def brute_positions(cu, T):
    """Walk the tokens one by one, counting up inside each sequence."""
    pos = [-1] * T
    for s in range(len(cu) - 1):
        n = 0
        for t in range(cu[s], cu[s + 1]):
            pos[t] = n
            n += 1
    return pos


def pin_positions(O):
    for cu, T in POSITION_CASES:
        got = O.segment_positions(np.array(cu, dtype=np.int32), T)
        assert list(got) == brute_positions(cu, T), (cu, list(got))


# ---------------------------------------------------------------------------
# frequencies, cos, sin
# ---------------------------------------------------------------------------

def pin_inv_freq(O):
    for theta in (1e4, 5e5, 1e6):
        for D in (2, 8, 64, 80, 128):
            got = O.inv_freq(theta, D)
            assert got.shape == (D // 2,)
            for i in range(D // 2):
                exact = mpmath.power(mpmath.mpf(theta), -mpmath.mpf(2 * i) / D)
                err = abs(mpmath.mpf(float(got[i])) - exact) / exact
                # one rounding of pow, plus the float64 rounding of the exponent 2i/D
                # (exact when D is a power of two) magnified by ln(theta)
                tol = F64_EPS + math.log(theta) * (2 * i / D) * 2.0 ** -53
                assert err <= tol, (theta, D, i, float(err))


def _exact_angle(p, theta, D, i):
    return mpmath.mpf(p) * mpmath.power(mpmath.mpf(theta), -mpmath.mpf(2 * i) / D)


def pin_cos_sin(O):
    """cos/sin at 50 digits; the only slack is the float64 rounding of the angle.

    |angle_f64 - angle| <= 1.5 ulp(angle) (one rounding in inv_freq scaled by
    p, one in the product), and cos/sin are 1-Lipschitz, plus one ulp of 1
    for the libm evaluation.
    """
    cases = [(0, 1e6, 64), (1, 1e6, 64), (151, 1e6, 64), (16383, 1e6, 64),
             (65535, 1e6, 128), (524287, 5e5, 128), (524287, 1e6, 128), (300000, 5e5, 128)]
    for p, theta, D in cases:
        for direction in (1, -1):
            c, s = O.cos_sin(np.array([p]), theta, D, direction)
            for i in range(0, D // 2, 3):
                a = _exact_angle(p, theta, D, i)
                tol = 1.5 * math.ulp(float(a)) + 2 * F64_EPS if p else 0.0
                ec = abs(mpmath.mpf(float(c[0, i])) - mpmath.cos(a))
                es = abs(mpmath.mpf(float(s[0, i])) - direction * mpmath.sin(a))
                assert ec <= tol and es <= tol, (p, theta, D, i, direction, float(ec), float(es))


# ---------------------------------------------------------------------------
# the rotation itself
# ---------------------------------------------------------------------------

def pin_closed_form_d2(O):
    """D = 2: inv_freq = [1], so (1,0) -> (cos p, sin p) and (0,1) -> (-sin p, cos p)."""
    ps = [0, 1, 2, 7, 100, 12345, 524287]
    T = len(ps)
    for theta in (1e4, 5e5):
        for direction in (1, -1):
            e1 = np.zeros((T, 1, 2))
            e1[:, 0, 0] = 1.0
            e2 = np.zeros((T, 1, 2))
            e2[:, 0, 1] = 1.0
            pos = np.array(ps)
            y1 = O.rotate(e1, pos, theta, direction)
            y2 = O.rotate(e2, pos, theta, direction)
            for r, p in enumerate(ps):
                c = mpmath.cos(p)
                s = direction * mpmath.sin(p)
                tol = 2 * F64_EPS
                assert abs(y1[r, 0, 0] - c) <= tol and abs(y1[r, 0, 1] - s) <= tol, (p, direction, y1[r])
                assert abs(y2[r, 0, 0] + s) <= tol and abs(y2[r, 0, 1] - c) <= tol, (p, direction, y2[r])


def _roformer_matrix(p, theta, D, direction):
    """RoFormer's rotary matrix for position p: 2x2 rotations on adjacent pairs
    (2i, 2i+1) by angle p * theta^(-2i/D), written out entry by entry."""
    R = [[mpmath.mpf(0)] * D for _ in range(D)]
    for i in range(D // 2):
        a = direction * _exact_angle(p, theta, D, i)
        c, s = mpmath.cos(a), mpmath.sin(a)
        R[2 * i][2 * i] = c
        R[2 * i][2 * i + 1] = -s
        R[2 * i + 1][2 * i] = s
        R[2 * i + 1][2 * i + 1] = c
    return R


def pin_roformer_matrix(O):
    """rotate_half RoPE == P^T R_adjacent P, where P interleaves (i, i+D/2) -> (2i, 2i+1)."""
    rng = _rng(11)
    for D, theta in ((8, 1e4), (12, 1e6), (16, 5e5)):
        ps = [0, 1, 5, 333, 90001]
        H = 2
        x = rng.standard_normal((len(ps), H, D))
        for direction in (1, -1):
            y = O.rotate(x, np.array(ps), theta, direction)
            for r, p in enumerate(ps):
                R = _roformer_matrix(p, theta, D, direction)
                for h in range(H):
                    z = [None] * D  # interleaved copy of the head
                    for i in range(D // 2):
                        z[2 * i] = mpmath.mpf(float(x[r, h, i]))
                        z[2 * i + 1] = mpmath.mpf(float(x[r, h, i + D // 2]))
                    w = [mpmath.fsum(R[a][b] * z[b] for b in range(D)) for a in range(D)]
                    norm = math.sqrt(sum(float(v) ** 2 for v in z))
                    tol = (8 * F64_EPS + 2 * math.ulp(float(_exact_angle(p, theta, D, 0)))) * max(norm, 1.0)
                    for i in range(D // 2):
                        assert abs(y[r, h, i] - w[2 * i]) <= tol, (D, p, h, i, direction)
                        assert abs(y[r, h, i + D // 2] - w[2 * i + 1]) <= tol, (D, p, h, i, direction)


def pin_complex_form(O):
    """(x_i + j x_{i+D/2}) * exp(j * direction * angle) in complex128."""
    rng = _rng(12)
    T, H, D, theta = 300, 3, 64, 1e6
    x = rng.standard_normal((T, H, D))
    pos = rng.integers(0, 524288, size=T)
    for direction in (1, -1):
        y = O.rotate(x, pos, theta, direction)
        i = np.arange(D // 2)
        # angles from mpmath-exact frequencies, rounded once to float64
        f = np.array([float(mpmath.power(mpmath.mpf(theta), -mpmath.mpf(2 * int(k)) / D)) for k in i])
        ang = pos[:, None].astype(np.float64) * f[None, :]
        rot = np.exp(1j * direction * ang)[:, None, :]
        z = (x[:, :, : D // 2] + 1j * x[:, :, D // 2:]) * rot
        scale = np.abs(x[:, :, : D // 2] + 1j * x[:, :, D // 2:])
        tol = 8 * F64_EPS * scale + 4 * F64_EPS * 524288 * scale  # angle rounding at positions up to 2^19
        assert np.all(np.abs(y[:, :, : D // 2] - z.real) <= tol)
        assert np.all(np.abs(y[:, :, D // 2:] - z.imag) <= tol)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def pin_identity_at_zero(O):
    rng = _rng(13)
    cu = np.array([0, 7, 40, 104, 256], dtype=np.int32)
    x = rng.standard_normal((256, 4, 64)).astype(np.float32).astype(np.float64)
    for direction in (1, -1):
        y = O.rope(x, cu, 1e6, direction)
        starts = cu[:-1]
        assert np.array_equal(y[starts], x[starts])


def pin_untouched_outside(O):
    rng = _rng(14)
    cu = np.array([3, 5, 5, 8], dtype=np.int32)
    x = rng.standard_normal((12, 2, 8))
    y = O.rope(x, cu, 1e4, 1)
    assert np.array_equal(y[:3], x[:3]) and np.array_equal(y[8:], x[8:])
    assert not np.array_equal(y[4], x[4])


def pin_pair_norm(O):
    rng = _rng(15)
    x = rng.standard_normal((500, 3, 128))
    pos = rng.integers(0, 524288, size=500)
    for direction in (1, -1):
        y = O.rotate(x, pos, 5e5, direction)
        n_in = x[:, :, :64] ** 2 + x[:, :, 64:] ** 2
        n_out = y[:, :, :64] ** 2 + y[:, :, 64:] ** 2
        assert np.all(np.abs(n_out - n_in) <= 1e-14 * np.maximum(n_in, 1e-300))


def pin_bwd_after_fwd(O):
    rng = _rng(16)
    cu = np.array([0, 100, 101, 1000, 4096], dtype=np.int32)
    x = rng.standard_normal((4096, 2, 64))
    y = O.rope(O.rope(x, cu, 1e6, 1), cu, 1e6, -1)
    assert np.max(np.abs(y - x)) <= 1e-14 * max(1.0, np.max(np.abs(x)))
    # and the other order
    y = O.rope(O.rope(x, cu, 1e6, -1), cu, 1e6, 1)
    assert np.max(np.abs(y - x)) <= 1e-14 * max(1.0, np.max(np.abs(x)))


def pin_relative_position(O):
    """<f(q, m), f(k, n)> depends on m - n only."""
    rng = _rng(17)
    D, theta = 64, 1e4
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    scale = np.linalg.norm(q) * np.linalg.norm(k)
    for m, n in ((5, 2), (100, 100), (3, 900), (1000, 10)):
        ref = np.sum(O.rotate(q, np.array([m]), theta, 1) * O.rotate(k, np.array([n]), theta, 1))
        for delta in (1, 17, 999, 9000):
            got = np.sum(O.rotate(q, np.array([m + delta]), theta, 1) * O.rotate(k, np.array([n + delta]), theta, 1))
            tol = 1e-12 * scale * max(1.0, (m + n + 2 * delta) / 1e4)
            assert abs(got - ref) <= tol, (m, n, delta, got, ref)
    # and it does depend on the difference
    a = np.sum(O.rotate(q, np.array([10]), theta, 1) * O.rotate(k, np.array([0]), theta, 1))
    b = np.sum(O.rotate(q, np.array([0]), theta, 1) * O.rotate(k, np.array([10]), theta, 1))
    assert abs(a - b) > 1e-6 * scale


def pin_packed_equals_unpacked(O):
    rng = _rng(18)
    lengths = [7, 1, 33, 0, 64, 151]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    x = rng.standard_normal((T, 3, 64))
    for direction in (1, -1):
        packed = O.rope(x, cu, 1e6, direction)
        for s, L in enumerate(lengths):
            a, b = int(cu[s]), int(cu[s + 1])
            alone = O.rope(x[a:b], np.array([0, L], dtype=np.int32), 1e6, direction)
            assert np.array_equal(packed[a:b], alone)


def pin_qk_share_angles(O):
    """q and k rotated by one call see the same positions and angles."""
    rng = _rng(19)
    cu = np.array([0, 10, 30], dtype=np.int32)
    q = rng.standard_normal((30, 4, 16))
    k = q[:, :2, :].copy()
    yq, yk = O.rope_qk(q, k, cu, 1e4, 1)
    assert np.array_equal(yq[:, :2, :], yk)


# ---------------------------------------------------------------------------
# variants: position offset, partial rotary dim, interleaved pairing, llama3 scaling
# ---------------------------------------------------------------------------

def pin_pos_offset_shards(O):
    """One sequence split over two token shards, the second with pos_offset = its
    global start, gives exactly the unsharded result; later segments of a shard
    keep restarting at 0."""
    rng = _rng(20)
    T, a = 300, 117
    x = rng.standard_normal((T, 2, 16))
    for direction in (1, -1):
        full = O.rope(x, [0, T], 1e4, direction)
        s1 = O.rope(x[:a], [0, a], 1e4, direction)
        s2 = O.rope(x[a:], [0, T - a], 1e4, direction, pos_offset=a)
        assert np.array_equal(np.concatenate([s1, s2]), full)
    # brute-force positions: the offset lands on segment 0 only
    for cu, T2 in (([0, 10, 50, 80], 90), ([4, 4, 9, 12], 12), ([0, 5], 5)):
        ref = brute_positions(cu, T2)
        for t in range(cu[0], cu[1]):
            ref[t] += 1000
        assert list(O.segment_positions(np.array(cu), T2, 1000)) == ref, cu
    # only segment 0 of a packed shard moves
    cu = np.array([0, 10, 50, 80], dtype=np.int32)
    x = rng.standard_normal((80, 2, 8))
    y0 = O.rope(x, cu, 1e4, 1)
    y1 = O.rope(x, cu, 1e4, 1, pos_offset=1000)
    assert np.array_equal(y0[10:], y1[10:]) and not np.array_equal(y0[:10], y1[:10])


def pin_rotary_dim(O):
    """rotary_dim r: elements [r, D) untouched; [0, r) is RoPE of a head of size r."""
    rng = _rng(21)
    cu = np.array([0, 13, 40], dtype=np.int32)
    x = rng.standard_normal((40, 3, 32))
    for r in (8, 16, 24):
        for pairing in ("half", "interleaved"):
            y = O.rope(x, cu, 1e4, 1, rotary_dim=r, pairing=pairing)
            assert np.array_equal(y[:, :, r:], x[:, :, r:])
            z = O.rope(np.ascontiguousarray(x[:, :, :r]), cu, 1e4, 1, pairing=pairing)
            assert np.array_equal(y[:, :, :r], z)


def pin_interleaved_roformer(O):
    """pairing='interleaved' is RoFormer's adjacent-pair matrix applied to the head as it is."""
    rng = _rng(22)
    for D, theta in ((8, 1e4), (12, 1e6)):
        ps = [0, 1, 5, 333, 90001]
        x = rng.standard_normal((len(ps), 2, D))
        for direction in (1, -1):
            y = O.rotate_interleaved(x, np.array(ps), O.inv_freq(theta, D), direction)
            for r, p in enumerate(ps):
                R = _roformer_matrix(p, theta, D, direction)
                for h in range(2):
                    z = [mpmath.mpf(float(v)) for v in x[r, h]]
                    w = [mpmath.fsum(R[a][b] * z[b] for b in range(D)) for a in range(D)]
                    norm = math.sqrt(sum(float(v) ** 2 for v in z))
                    tol = (8 * F64_EPS + 2 * math.ulp(float(_exact_angle(p, theta, D, 0)))) * max(norm, 1.0)
                    for i in range(D):
                        assert abs(y[r, h, i] - w[i]) <= tol, (D, p, h, i, direction)
    # the packed call takes the same route
    cu = np.array([0, 5], dtype=np.int32)
    x = rng.standard_normal((5, 2, 8))
    ya = O.rope(x, cu, 1e4, 1, pairing="interleaved")
    yb = O.rotate_interleaved(x, np.arange(5), O.inv_freq(1e4, 8), 1)
    assert np.array_equal(ya, yb)


def pin_llama3_scaling(O):
    """Properties of the Llama 3.1 frequency rescaling (no retyped formula):
    factor 1 is the identity; with every wavelength above the band all
    frequencies are divided by the factor, below it none are; the rescaled
    frequency is continuous at both band edges, linear in L / wavelength
    inside the band, and decreasing in i like the unscaled frequencies."""
    theta, D = 5e5, 128
    base = O.inv_freq(theta, D)
    kw = dict(low_freq_factor=1.0, high_freq_factor=4.0, original_max_position=8192.0)
    same = O.llama3_inv_freq(theta, D, factor=1.0, **kw)
    assert np.all(np.abs(same - base) <= 2 * F64_EPS * base)
    tiny_L = O.llama3_inv_freq(theta, D, factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0, original_max_position=1e-9)
    assert np.all(np.abs(tiny_L - base / 8.0) <= F64_EPS * base)  # every wavelength is above L / low_freq_factor
    huge_L = O.llama3_inv_freq(theta, D, factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0, original_max_position=1e12)
    assert np.array_equal(huge_L, base)  # every wavelength is below L / high_freq_factor
    got = O.llama3_inv_freq(theta, D, factor=8.0, **kw)
    assert np.all(np.diff(got) < 0)
    # ratio got/base as a function of u = L / wavelength (wavelength = 2 pi / f)
    u = kw["original_max_position"] * base / (2 * math.pi)
    ratio = got / base
    band = (u > 1.0) & (u < 4.0)
    assert band.sum() >= 3, "the test needs frequencies inside the band"
    assert np.all(np.abs(ratio[u >= 4.0 + 1e-9] - 1.0) <= 2 * F64_EPS)
    assert np.all(np.abs(ratio[u <= 1.0 - 1e-9] - 1.0 / 8.0) <= 2 * F64_EPS)
    # continuity: extrapolating the band's line to u = 1 and u = 4 meets 1/8 and 1
    ub, rb = u[band], ratio[band]
    slope, icpt = np.polyfit(ub, rb, 1)
    assert np.max(np.abs(slope * ub + icpt - rb)) <= 1e-13  # linear in u inside the band
    assert abs(slope * 1.0 + icpt - 1.0 / 8.0) <= 1e-12 and abs(slope * 4.0 + icpt - 1.0) <= 1e-12


# float32-convention angles, worked by hand in exact rational arithmetic
# (theta = 1e6, D = 128): (pair i, position, the float32 angle, and for
# contrast the angle with only the frequency rounded, with only the product
# rounded, and the float64 angle).  i = 0 has frequency 1, so its float32
# angle is the position rounded to float32 (2^24 + 1 is a tie, to even).
FP32_ANGLE_CASES = [
    (1, 77777, 62675.984375, 62675.985769987106, 62675.98828125, 62675.98783752477),
    (31, 77777, 96.51641082763672, 96.51641442882828, 96.51641845703125, 96.51641621798649),
    (0, 2 ** 24 + 1, 16777216.0, 16777217.0, 16777216.0, 16777217.0),
    (0, 2 ** 24 + 3, 16777220.0, 16777219.0, 16777220.0, 16777219.0),
    (31, 2 ** 24 + 1, 20819.48046875, 20819.481709687738, 20819.482421875, 20819.48209562568),  # position rounded first
]


def pin_fp32_freq_angles(O):
    """freq_precision='fp32': the hand-worked angles above (a unit vector in
    pair i rotates to (cos a, sin a)); a power-of-two base whose frequencies
    and products are exact in float32 gives the float64 result bit for bit;
    elsewhere the angles move by at most two float32 roundings (2^-23
    relative), and do move."""
    theta, D = 1e6, 128
    for i, p, a32, *_ in FP32_ANGLE_CASES:
        for pairing in ("half", "interleaved"):
            x = np.zeros((1, 1, D))
            j1, j2 = (i, i + D // 2) if pairing == "half" else (2 * i, 2 * i + 1)
            x[0, 0, j1] = 1.0
            y = O.rope(x, [0, 1], theta, 1, pos_offset=p, pairing=pairing, freq_precision="fp32")
            assert abs(y[0, 0, j1] - math.cos(a32)) <= 4 * F64_EPS, (i, p, pairing)
            assert abs(y[0, 0, j2] - math.sin(a32)) <= 4 * F64_EPS, (i, p, pairing)
    rng = _rng(23)
    x = rng.standard_normal((64, 2, 4))
    for off in (0, 2 ** 24 - 64):  # theta = 2^16, D = 4: frequencies 1 and 2^-8
        a = O.rope(x, [0, 64], 2.0 ** 16, 1, pos_offset=off, freq_precision="fp32")
        b = O.rope(x, [0, 64], 2.0 ** 16, 1, pos_offset=off)
        assert np.array_equal(a, b), off
    pos = rng.integers(0, 2 ** 21, size=300)
    x = rng.standard_normal((300, 1, D))
    ys = []
    for fp in ("fp32", "fp64"):
        ys.append(np.stack([O.rope(x[n:n + 1], [0, 1], theta, 1, pos_offset=int(pos[n]), freq_precision=fp)[0]
                            for n in range(300)]))
    y32, y64 = ys
    ang_max = pos.astype(np.float64)[:, None] * O.inv_freq(theta, D)[None, :]  # [N, D/2]
    norm = np.hypot(x[:, 0, : D // 2], x[:, 0, D // 2:])
    bound = norm * ang_max * 2.0 ** -23 * 1.01 + 1e-12
    dev = np.hypot(y32[:, 0, : D // 2] - y64[:, 0, : D // 2], y32[:, 0, D // 2:] - y64[:, 0, D // 2:])
    assert np.all(dev <= bound)
    assert np.count_nonzero(dev > 1e-9) > 100


ALL_PINS = [
    pin_positions,
    pin_inv_freq,
    pin_cos_sin,
    pin_closed_form_d2,
    pin_roformer_matrix,
    pin_complex_form,
    pin_identity_at_zero,
    pin_untouched_outside,
    pin_pair_norm,
    pin_bwd_after_fwd,
    pin_relative_position,
    pin_packed_equals_unpacked,
    pin_qk_share_angles,
    pin_pos_offset_shards,
    pin_rotary_dim,
    pin_interleaved_roformer,
    pin_llama3_scaling,
    pin_fp32_freq_angles,
]
