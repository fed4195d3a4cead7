"""The source fold divides by a scale without a float64 division per element: with rs the correctly
rounded 1/s, q = RN(v * rs), the exact residual r = RN(v - q * s) (one fused multiply-add) and
q' = RN(q + r * rs) (another) give the correctly rounded quotient v / s (Markstein's theorem on
division by multiplication). The fold stores that quotient rounded to float32, so its output is
bit-identical to the exact division's. This checks the arithmetic on the CPU, emulating each fused
multiply-add exactly with rationals, on random operands in the fold's input range
(float32 values, positive scales between 2^-500 and 2^500)."""
from fractions import Fraction

import numpy as np
import pytest


def _fma(a: float, b: float, c: float) -> float:
    return float(Fraction(a) * Fraction(b) + Fraction(c))  # one rounding, to nearest even


def _markstein(v: float, s: float) -> float:
    rs = 1.0 / s
    q = v * rs
    r = _fma(-q, s, v)
    return _fma(r, rs, q)


def _operands(rng, n):
    v = rng.standard_normal(n).astype(np.float32) * np.float32(2.0) ** rng.integers(-60, 60, n).astype(np.float32)
    s = np.exp(rng.uniform(np.log(1e-4), np.log(1e4), n))
    return v.astype(np.float64), s


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quotient_is_correctly_rounded(seed):
    rng = np.random.default_rng(seed)
    v, s = _operands(rng, 4000)
    for a, b in zip(v.tolist(), s.tolist()):
        assert _markstein(a, b) == a / b


def test_extreme_scales_and_subnormal_float32_inputs():
    rng = np.random.default_rng(7)
    vals = [float(np.float32(1e-45)), float(np.float32(-3e-42)), float(np.finfo(np.float32).max), -1.5, 3.0]
    for e in (-500, -499, -200, -3, 0, 5, 300, 500):
        for a in vals:
            for m in (1.0, 1.5, 1.9999999999999998, 1.3333333333333333):
                b = m * 2.0 ** e
                assert _markstein(a, b) == a / b
    # random scales across the whole range
    for _ in range(3000):
        a = float(np.float32(rng.standard_normal() * 2.0 ** rng.integers(-126, 127)))
        b = float(rng.uniform(1, 2) * 2.0 ** rng.integers(-500, 500))
        assert _markstein(a, b) == a / b


def test_correction_step_is_needed():
    """On random operands the plain product v * rs is sometimes one ulp off the quotient; the
    corrected value never is."""
    rng = np.random.default_rng(11)
    wrong_product = 0
    for _ in range(4000):
        b = float(rng.uniform(1, 2) * 2.0 ** rng.integers(-20, 20))
        a = float(np.float32(rng.standard_normal()))
        if a == 0.0:
            continue
        want = a / b
        assert _markstein(a, b) == want
        wrong_product += a * (1.0 / b) != want
    # the plain product is not always correct: the correction step matters
    assert wrong_product > 0
