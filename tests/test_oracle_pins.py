"""The CPU oracle against what the pages and mathematics fix (no GPU needed)."""
from fractions import Fraction

import numpy as np
import pytest

from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle, pin):
    pin(oracle)


def test_exact_quotient_reference():
    """The integer-arithmetic rounding used by the exact pins, against two independent
    routes: Python's Fraction with a nearest-neighbour search (every case), and the
    float64 quotient or product rounded to binary32 (correct, because a binary32
    result computed to 53 bits and rounded again is never double-rounded wrongly:
    53 >= 2 * 24 + 2)."""
    rng = np.random.default_rng(71)
    a = np.concatenate([pins.random_f32(3000, 72, -149, 127), np.float32([1.0, -3.0, 1e-45, 3.4e38, 0.0, -0.0])])
    b = np.concatenate([pins.random_f32(3000, 73, -149, 127), np.float32([3.0, 7.0, 2.0, 0.5, 5.0, -5.0])])
    a = a[np.isfinite(a)][: b.size]
    b = b[: a.size]
    with np.errstate(over="ignore", under="ignore"):
        d64 = (a.astype(np.float64) / b.astype(np.float64)).astype(np.float32)
        m64 = (a.astype(np.float64) * b.astype(np.float64)).astype(np.float32)
    d = pins.rn_div_f32(a, b)
    m = pins.rn_mul_f32(a, b)
    assert np.array_equal(pins.f32_bits(d), pins.f32_bits(d64))
    assert np.array_equal(pins.f32_bits(m), pins.f32_bits(m64))
    for i in rng.choice(a.size, 400, replace=False):
        x, y = Fraction(float(a[i])), Fraction(float(b[i]))
        q = x / y
        if q != 0 and abs(q) < Fraction(3.4e38):
            assert pins.f32_bits(pins.rn_f32_of(q)) == pins.f32_bits(d[i]), (a[i], b[i])
    # exact ties go to the even significand, at normal and subnormal magnitudes
    assert pins.rn_f32_ratio((1 << 24) + 1, 1 << 24) == 1.0
    assert pins.rn_f32_ratio((1 << 24) + 3, 1 << 24) == 1.0 + 2.0 ** -22
    assert pins.rn_f32_ratio(1, 1 << 150) == 0.0 and pins.rn_f32_ratio(3, 1 << 150) == 2.0 ** -148
    assert pins.rn_f32_ratio(-1, 1 << 151) == 0.0 and np.signbit(pins.rn_f32_ratio(-1, 1 << 151))
    assert pins.rn_f32_ratio(1 << 128, 1) == float("inf")
