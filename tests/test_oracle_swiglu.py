"""Pins for the oracle's SwiGLU epilogue (not GPU).

"Development Guide for Small AI Models (TinyLLaMA, etc.) Using C++", §4.4:
SwiGLU(x) = Swish(x W_gate) * (x W_up) elementwise, Swish(z) = z sigma(z),
sigma(z) = 1 / (1 + e^{-z}).

Pinned by closed forms (sigma(ln 3) = 3/4, sigma(-ln 3) = 1/4), the identity
Swish(z) - Swish(-z) = z (from sigma(z) + sigma(-z) = 1), the series
Swish(z) = z/2 + z^2/4 + O(z^4) near zero, the limits at both ends, and
the stationary point: where Swish' = 0, sigma = 1 + 1/z and so Swish = z + 1.
A flipped exponent sign, a dropped factor z or a wrong operand of the
product fails one of them.
"""
import math

import numpy as np


def test_swish_closed_forms(orc):
    l3 = math.log(3.0)
    assert math.isclose(orc.swish(l3), 0.75 * l3, rel_tol=1e-15)
    assert math.isclose(orc.swish(-l3), -0.25 * l3, rel_tol=1e-15)
    assert orc.swish(0.0) == 0.0
    # sigma(ln 7) = 7/8
    l7 = math.log(7.0)
    assert math.isclose(orc.swish(l7), 0.875 * l7, rel_tol=1e-15)


def test_swish_odd_part_identity(orc):
    zs = np.random.default_rng(3).uniform(-30.0, 30.0, 2000)
    for z in zs:
        d = orc.swish(z) - orc.swish(-z)
        assert abs(d - z) <= 4e-16 * abs(z) + 1e-300, z


def test_swish_series_near_zero(orc):
    for z in (1e-3, -1e-3, 1e-6, -2.5e-5, 1e-9):
        approx = z / 2 + z * z / 4          # next term is -z^4/48
        assert abs(orc.swish(z) - approx) <= abs(z) ** 4 / 40 + 2e-16 * abs(z), z


def test_swish_limits(orc):
    assert orc.swish(40.0) == 40.0               # 1 + e^-40 rounds to 1
    assert orc.swish(745.0) == 745.0
    t = orc.swish(-40.0)                         # -40 e^-40 / (1 + e^-40)
    assert math.isclose(t, -40.0 * math.exp(-40.0), rel_tol=1e-15)
    big = orc.swish(-1000.0)                     # e^1000 overflows: the limit -0
    assert big == 0.0 and math.copysign(1.0, big) < 0


def test_swish_stationary_point(orc):
    """Bisection on the oracle's own finite-difference slope locates the
    minimum; there Swish(z*) must equal z* + 1 (and z* ~ -1.27846)."""
    def slope(z, h=1e-6):
        return (orc.swish(z + h) - orc.swish(z - h)) / (2 * h)
    lo, hi = -2.0, -0.5
    assert slope(lo) < 0 < slope(hi)
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        if slope(mid) < 0:
            lo = mid
        else:
            hi = mid
    z = 0.5 * (lo + hi)
    assert abs(z + 1.2784645) < 1e-5
    assert abs(orc.swish(z) - (z + 1.0)) < 1e-9


def test_swiglu_elementwise(orc):
    l3 = math.log(3.0)
    g = np.array([l3, -l3, 0.0, 40.0, -1000.0, 2.0])
    u = np.array([4.0, 8.0, 5.0, -0.5, 3.0, 0.0])
    h = orc.swiglu(g, u)
    expect = [3.0 * l3, -2.0 * l3, 0.0, -20.0, 0.0, 0.0]
    for got, e in zip(h, expect):
        assert math.isclose(got, e, rel_tol=1e-15, abs_tol=1e-300)
    # shapes are kept and the product is elementwise
    g2 = np.random.default_rng(5).standard_normal((3, 7))
    u2 = np.random.default_rng(6).standard_normal((3, 7))
    h2 = orc.swiglu(g2, u2)
    assert h2.shape == (3, 7)
    for i in range(3):
        for j in range(7):
            assert h2[i, j] == orc.swish(g2[i, j]) * u2[i, j]
