"""The kernel's float64 sin/cos (csrc/rope_sincos.h), built for the host, against mpmath.

The HIP kernels evaluate cos/sin of position * inv_freq with their own
Cody-Waite reduction and Taylor series.  The same source compiles for the
host, so its accuracy is checked here on the CPU over the whole angle range
the kernels see (0 <= angle < 2^31), including arguments next to multiples
of pi/2 where the reduction loses the most.
"""

import os
import subprocess

import mpmath
import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR_DIR = os.path.join(ROOT, "packed_varlen_rotary_amd", "csrc")

DRIVER = r"""
#include <stdio.h>
#include <stdlib.h>
#include "rope_sincos.h"
int main(void) {
  double x;
  while (scanf("%la", &x) == 1) {
    double s, c;
    rope_sincos(x, &s, &c);
    printf("%a %a\n", s, c);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    d = tmp_path_factory.mktemp("sincos")
    src = d / "driver.c"
    src.write_text(DRIVER)
    exe = d / "driver"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-I", HDR_DIR, str(src), "-o", str(exe), "-lm"], check=True)
    return str(exe)


def run(driver, xs):
    inp = "\n".join(float(x).hex() for x in xs) + "\n"
    out = subprocess.run([driver], input=inp, capture_output=True, text=True, check=True).stdout.split()
    v = [float.fromhex(t) for t in out]
    return np.array(v[0::2]), np.array(v[1::2])


def arguments():
    rng = np.random.default_rng(3)
    xs = [0.0, 1.0, 0.5, 1e-8, 2.0 ** -30]
    xs += list(rng.uniform(0, 10, 300))
    xs += list(rng.uniform(0, 524288, 300))
    xs += list(rng.uniform(0, 2.0 ** 31, 300))
    # angles the kernels form: position * theta^(-2i/D)
    for theta, D in ((1e6, 64), (1e6, 128), (5e5, 128)):
        f = theta ** (-(2.0 * np.arange(D // 2)) / D)
        pos = rng.integers(0, 524288, 64).astype(np.float64)
        xs += list((pos[:, None] * f[None, :]).ravel()[::7])
    # float64 neighbours of multiples of pi/2 (the reduction's hardest inputs)
    mpmath.mp.dps = 40
    for k in list(range(1, 40)) + [int(v) for v in rng.integers(1, 1_300_000_000, 60)]:
        m = float(k * mpmath.pi / 2)
        xs += [m, np.nextafter(m, 0), np.nextafter(m, np.inf)]
    return [x for x in xs if 0 <= x < 2.0 ** 31]


def test_rope_sincos_accuracy(driver):
    xs = arguments()
    s, c = run(driver, xs)
    mpmath.mp.dps = 50
    worst = 0.0
    for x, si, ci in zip(xs, s, c):
        es = abs(mpmath.mpf(si) - mpmath.sin(mpmath.mpf(x)))
        ec = abs(mpmath.mpf(ci) - mpmath.cos(mpmath.mpf(x)))
        worst = max(worst, float(es), float(ec))
    # a few units of 2^-53 in absolute terms over the whole range
    assert worst <= 4 * 2.0 ** -53, worst


def test_rope_sincos_exact_at_zero(driver):
    s, c = run(driver, [0.0])
    assert s[0] == 0.0 and c[0] == 1.0
