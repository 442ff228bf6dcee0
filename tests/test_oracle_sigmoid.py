"""Pins for the oracle's sigmoid (CPU only).

The pass needs sigmoid(gate) for bf16 gates only, so every one of the 65,280
finite bf16 values is checked.  The oracle computes e = fp32(exp(-g)),
den = 1 + e, s = 1 / den in fp32 (a reading: the page asks for the SwiGLU
gradient without fixing how sigmoid is evaluated).  Pinned here:

* e is the correctly rounded fp32 value of exp(-g), against 60-digit decimal
  exponentials rounded by the exact rounding rule in ``tests/exact.py``;
* s is within the error bound of three correctly rounded steps of the true
  sigmoid, |s - sigma(g)| <= 3 * 2^-24 * sigma(g) + 2^-150;
* the closed forms the fp32 evaluation must have: s(0) = 1/2 exactly, s == 1
  from g = 16.75 up, s == 0 from g = -89 down, s == 1/2 for tiny |g|, and s is
  monotone non-decreasing in g.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact import all_finite_bf16, bf16_bits_to_fraction, exp_exact, rn32, sigmoid_exact

BF16 = all_finite_bf16()


def _bits_to_float(b):
    return float(bf16_bits_to_fraction(int(b)))


@pytest.fixture(scope="module")
def oracle_table():
    """(g, e, den, s) of the oracle for every finite bf16 gate."""
    rows = []
    for b in BF16:
        g = _bits_to_float(b)
        e, den, s = oracle.sigmoid_parts(g)
        rows.append((g, float(e), float(den), float(s)))
    return rows


def test_exp_is_correctly_rounded(oracle_table):
    """e must be the fp32 nearest to exp(-g) for every finite bf16 g."""
    bad = []
    for g, e, _, _ in oracle_table:
        if g > 110.0:  # exp(-g) < 2^-158: below half the smallest subnormal
            want = 0.0
        elif g < -100.0:  # exp(-g) > 2^144: beyond the fp32 range
            want = float("inf")
        else:
            r = rn32(exp_exact(-Fraction(g)))
            want = float(r)
        if e != want:
            bad.append((g, e, want))
    assert not bad, "exp(-g) misrounded for %d gates, e.g. %r" % (len(bad), bad[:5])


def test_sigmoid_within_three_roundings_of_exact(oracle_table):
    bound_rel = Fraction(3, 2**24)
    tiny = Fraction(1, 2**150)
    worst = Fraction(0)
    flt_max = (2 - Fraction(1, 2**23)) * Fraction(2) ** 127
    for g, e, _, s in oracle_table:
        if abs(g) > 120.0:
            exact = Fraction(1) if g > 0 else Fraction(0)
        else:
            exact = sigmoid_exact(Fraction(g))
        err = abs(Fraction(s) - exact)
        if e == float("inf"):
            # exp(-g) overflowed fp32: the evaluation gives 0, and the true
            # sigmoid is below 1/FLT_MAX there.
            assert s == 0.0 and exact < 1 / flt_max, g
            continue
        assert err <= bound_rel * exact + tiny, (g, s, float(exact))
        if exact > 0:
            worst = max(worst, err / exact)
    assert worst > 0  # the check really compared something


def test_sigmoid_closed_forms(oracle_table):
    for g, e, den, s in oracle_table:
        if g == 0.0:
            assert s == 0.5 and e == 1.0 and den == 2.0
        if g >= 16.75:
            # exp(-16.75) < 2^-24, so 1 + e rounds to 1
            assert s == 1.0, g
        if g <= -89.0:
            # exp(89) > FLT_MAX, so e = inf and s = 1/inf = 0
            assert e == float("inf") and s == 0.0, g
        if 0.0 <= g <= 8.9e-8 or -1.78e-7 <= g <= 0.0:
            # 1 + e is within half an ulp of 2 on these ranges
            assert s == 0.5, g
    by_g = {g: s for g, _, _, s in oracle_table}
    assert by_g[16.625] < 1.0  # exp(-16.625) > 2^-24 still moves 1 + e
    assert 0.0 < by_g[-88.5] < 2.0**-126  # subnormal sigmoid, kept (no flush)


def test_sigmoid_monotone(oracle_table):
    pts = sorted((g, s) for g, _, _, s in oracle_table)
    ss = np.array([s for _, s in pts])
    assert np.all(np.diff(ss) >= 0)


def test_nontrivial_gate_count(oracle_table):
    """Only 7,223 finite bf16 gates give s outside {0, 1/2, 1}; the rest
    saturate or sit at the midpoint."""
    n = sum(1 for _, _, _, s in oracle_table if s not in (0.0, 0.5, 1.0))
    assert n == 7223
