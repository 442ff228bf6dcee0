"""Pins for the oracle's group quantiser (CPU only).

The quantiser (scale = amax / 127, 1.0 for an all-zero group; inv = 1 / scale;
q = clamp(rne(v * inv), -127, 127)) is pinned by:

* the rounding rule itself: each code is the integer nearest (ties to even)
  to the fp32 product RN(v * inv), both roundings done here in exact rational
  arithmetic, including a hand-derived group where rounding the exact product
  instead would give a different code (tests/golden/quant_worked_examples.txt,
  ``fp32_product_tie``) and a search that finds such groups;
* hand-derived worked examples whose exact results are known without running
  any float code (the fixture tests/golden/quant_worked_examples.txt, with the
  derivations and the rules they follow);
* brute-force rounding: with amax = 127 the scale and its inverse are exactly 1,
  so every code must be the integer nearest to v (ties to even), found here by
  comparing the two integer neighbours in exact arithmetic, for every bf16
  value in [-127, 127];
* invariants on random groups: |q| <= 127, some |q| == 127 in every group with
  a normal-range scale, zero groups give scale 1.0 and zero codes, signs agree,
  codes are monotone in v, and the dequantised error is at most half a scale
  step plus the rounding slack of inv and v * inv.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact import all_finite_bf16, bf16_bits_to_fraction, f32_bits, rn32, rne_int


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "quant_worked_examples.txt")


def _worked_examples():
    rows = []
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            name, values, bits, codes = (f.strip() for f in line.split("|"))
            rows.append((name, [float(v) for v in values.split()], int(bits, 16), [int(c) for c in codes.split()]))
    return rows


@pytest.mark.parametrize("name,values,bits,codes", _worked_examples(), ids=lambda v: v if isinstance(v, str) else "")
def test_worked_examples(name, values, bits, codes):
    # derivations in tests/golden/quant_worked_examples.txt
    q, s = oracle.quant_group(values)
    assert f32_bits(s) == bits, name
    assert q.tolist() == codes, name


def test_worked_examples_are_all_there():
    assert [r[0] for r in _worked_examples()] == ["amax_one", "amax_127_ties", "fp32_product_tie"]


def test_zero_group():
    q, s = oracle.quant_group([0.0] * 128)
    assert s == 1.0 and not q.any()
    q, s = oracle.quant_group([-0.0] * 5)
    assert s == 1.0 and not q.any()


def test_brute_force_rounding_all_bf16_in_range():
    bits = all_finite_bf16()
    vals = np.array([float(bf16_bits_to_fraction(int(b))) for b in bits], dtype=np.float64)
    vals = vals[np.abs(vals) <= 127.0]
    group = np.concatenate([[127.0], vals]).astype(np.float32)
    q, s = oracle.quant_group(group)
    assert s == 1.0
    for v, code in zip(group, q):
        assert int(code) == rne_int(Fraction(float(v))), (float(v), int(code))


def test_tiny_scale_overflowing_inverse():
    # amax = 2^-130 (a bf16 subnormal): scale = 2^-130/127 is a subnormal fp32
    # and 1/scale overflows to +inf.  Zeros stay 0, non-zeros clamp to +-127.
    tiny = 2.0**-130
    q, s = oracle.quant_group([tiny, -tiny, 0.0, tiny / 2])
    assert Fraction(float(s)) == rn32(Fraction(tiny) / 127)
    assert q.tolist() == [127, -127, 0, 127]


def _random_groups(rng, n_groups=400):
    groups = []
    for i in range(n_groups):
        n = int(rng.integers(1, 129))
        mag = 10.0 ** rng.uniform(-30, 30)
        v = rng.standard_normal(n) * mag
        if i % 7 == 0:
            v[rng.integers(0, n, size=max(1, n // 4))] = 0.0
        # bf16-representable values, as the pass produces
        v = np.array([float(bf16_bits_to_fraction(oracle.f32_to_bf16(float(x)))) for x in v])
        groups.append(v.astype(np.float32))
    return groups


def test_invariants_random_groups():
    rng = np.random.default_rng(7)
    for v in _random_groups(rng):
        q, s = oracle.quant_group(v)
        qi = q.astype(np.int64)
        amax = float(np.max(np.abs(v)))
        assert np.all(np.abs(qi) <= 127)
        if amax == 0.0:
            assert s == 1.0 and not q.any()
            continue
        assert Fraction(float(s)) == rn32(Fraction(amax) / 127)
        if float(s) >= 2.0**-126:
            assert np.max(np.abs(qi)) == 127
        # sign agreement and zeros
        assert np.all((qi == 0) | (np.sign(qi) == np.sign(v)))
        assert np.all(qi[v == 0] == 0)
        # monotone in v
        order = np.argsort(v, kind="stable")
        assert np.all(np.diff(qi[order]) >= 0)
        # dequantisation error bound, in double
        err = np.abs(qi * float(s) - v.astype(np.float64))
        assert np.all(err <= float(s) * (0.5 + 2.0**-15)), (err.max(), float(s))


def _inv_of(scale) -> Fraction:
    return rn32(1 / Fraction(float(scale)))


def test_codes_round_the_fp32_product():
    rng = np.random.default_rng(11)
    for v in _random_groups(rng, n_groups=150):
        q, s = oracle.quant_group(v)
        if float(np.max(np.abs(v))) == 0.0 or float(s) < 2.0**-126:
            continue
        inv = _inv_of(s)
        for x, code in zip(v, q):
            want = max(-127, min(127, rne_int(rn32(Fraction(float(x)) * inv))))
            assert int(code) == want, (float(x), float(s), int(code), want)


def _double_rounding_cases(limit=None):
    """Groups (amax, v) where the fp32 product RN(v * inv) is a tie k + 1/2
    that the exact product v * inv is not on, so rounding the product to fp32
    first gives a different code than rounding the exact product."""
    cases = []
    for num in range(129, 256):
        amax = Fraction(num, 2)  # bf16-exact values in (64, 128)
        inv = rn32(1 / rn32(amax / 127))
        for vnum in range(1, 256):
            v = Fraction(vnum, 4)
            if v > amax:
                break
            exact = v * inv
            via_f32 = rn32(exact)
            if rne_int(exact) != rne_int(via_f32):
                cases.append((amax, v, rne_int(via_f32), rne_int(exact)))
                if limit and len(cases) >= limit:
                    return cases
    return cases


def test_fp32_product_not_the_exact_product():
    cases = _double_rounding_cases(limit=20)
    assert len(cases) == 20
    for amax, v, want, other in cases:
        q, s = oracle.quant_group([float(amax), float(v)])
        assert int(q[0]) == 127
        assert int(q[1]) == want != other, (amax, v)
