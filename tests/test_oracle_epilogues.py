"""Pins of the oracle's SwiGLU activation (oracle.swiglu), the reference of the
GEMV's SwiGLU epilogue: silu(g) * u with silu(g) = g / (1 + exp(-g)).

Closed forms (silu(0) = 0, silu(g) - silu(-g) = g, the large-|g| limits, the
value at g = ln 3 where the sigmoid is 3/4) and a scalar evaluation with the
standard library's exp in exact rational arithmetic around it."""
import math
from fractions import Fraction

import numpy as np

import oracle


def test_closed_forms():
    u = np.array([1.5, -2.0, 3.0])
    assert np.all(oracle.swiglu(np.zeros(3), u) == 0)
    g = np.array([0.3, 1.7, 12.0, 80.0])
    d = oracle.swiglu(g, np.ones(4)) - oracle.swiglu(-g, np.ones(4))
    assert np.allclose(d, g, rtol=1e-15, atol=0)
    assert oracle.swiglu(np.array([60.0]), np.array([2.0]))[0] == 120.0
    assert abs(oracle.swiglu(np.array([-60.0]), np.array([2.0]))[0]) < 1e-23
    # sigmoid(ln 3) = 3/4
    assert abs(oracle.swiglu(np.array([math.log(3.0)]), np.array([4.0]))[0] - 3.0 * math.log(3.0)) < 1e-15


def test_scalar_reference():
    r = np.random.default_rng(0)
    g = r.standard_normal(200) * 6
    u = r.standard_normal(200) * 3
    h = oracle.swiglu(g, u)
    for gi, ui, hi in zip(g, u, h):
        ref = Fraction(gi) / (1 + Fraction(math.exp(-gi))) * Fraction(ui)
        assert abs(Fraction(hi) - ref) <= abs(ref) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 1000)
