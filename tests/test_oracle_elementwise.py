"""Pins for the oracle's elementwise part and its bf16 rounding (CPU only).

* The gradient formula is checked against central finite differences of the
  forward function f(g, u) = silu(g) * u, taken in double precision from the
  forward function alone (so a dropped term, a wrong sign or a swapped operand
  in the backward formula shows up as a gross mismatch).
* y, d_gate and d_up before rounding are within a few fp32 roundings of the
  exact values.
* bf16 rounding agrees with PyTorch's own float32 -> bfloat16 conversion (a
  library routine, round to nearest even) on random bit patterns, ties and
  subnormals.
"""

import math

import numpy as np
import pytest
import torch

import oracle


def _f(g, u):
    return g / (1.0 + math.exp(-g)) * u


def _fd_dg(g, u, h=1e-5):
    return (_f(g + h, u) - _f(g - h, u)) / (2 * h)


def _fd_du(g, u, h=1e-5):
    return (_f(g, u + h) - _f(g, u - h)) / (2 * h)


GATES = list(np.linspace(-6.0, 6.0, 13)) + [-11.5, -2.75, -1.28125, -0.3125, 0.15625, 3.375, 9.0, 14.5]
UPS = [0.7, -1.3, 2.5, 0.0078125]
DYS = [1.0, 0.01, -3.0]


@pytest.mark.parametrize("d", DYS)
@pytest.mark.parametrize("u", UPS)
def test_gradients_match_finite_differences(u, d):
    for g in GATES:
        g32, u32, d32 = (float(np.float32(v)) for v in (g, u, d))
        y, dg, du = oracle.pair_f32(g32, u32, d32)
        want_dg = d32 * _fd_dg(g32, u32)
        want_du = d32 * _fd_du(g32, u32)
        want_y = _f(g32, u32)
        # finite differences are good to ~1e-10 relative here; fp32 evaluation to
        # a few ulps.  Scale the tolerance by the size of the factors involved.
        tol_dg = 2e-6 * abs(d32 * u32) * (1.0 + abs(g32)) + 1e-12
        assert abs(float(dg) - want_dg) <= tol_dg, (g, u, d, dg, want_dg)
        assert abs(float(du) - want_du) <= 2e-6 * abs(d32 * g32) + 1e-12, (g, u, d, du, want_du)
        assert abs(float(y) - want_y) <= 2e-6 * abs(g32 * u32) + 1e-12, (g, u, y, want_y)


def test_gradient_sign_and_zero_of_dgate():
    # d/dg silu(g) = s * (1 + g * (1 - s)) crosses zero near g = -1.2785 and is
    # negative just below it.
    _, dg_lo, _ = oracle.pair_f32(-1.5, 1.0, 1.0)
    _, dg_hi, _ = oracle.pair_f32(-1.0, 1.0, 1.0)
    assert dg_lo < 0 < dg_hi


def _torch_bf16_bits(f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(f32.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # exact ties (low half 0x8000), one below/above, and subnormals
    ties = (rng.integers(0, 2**16, size=20_000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    near = np.concatenate([ties - 1, ties + 1])
    sub = rng.integers(0, 0x00800000, size=20_000, dtype=np.uint64).astype(np.uint32)
    sub = np.concatenate([sub, sub | 0x80000000])
    allbits = np.concatenate([bits, ties, near, sub])
    f = allbits.view(np.float32)
    keep = ~np.isnan(f) & ~np.isnan(_torch_bits_to_f32(_torch_bf16_bits(f)))
    f = f[keep]
    want = _torch_bf16_bits(f)
    got = np.array([oracle.f32_to_bf16(float(v)) for v in f], dtype=np.uint16)
    mismatch = np.nonzero(got != want)[0]
    assert mismatch.size == 0, [(hex(f.view(np.uint32)[i]), hex(got[i]), hex(want[i])) for i in mismatch[:5]]


def _torch_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def test_bf16_widening_is_exact():
    for b in (0x0000, 0x8000, 0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x4186, 0xC2B2):
        assert oracle.bf16_to_f32(b) == float(_torch_bits_to_f32(np.array([b], dtype=np.uint16))[0])
