"""Pins for the oracle's FP8 (OCP E4M3) variant (CPU only).

* Decoding: the bit patterns with closed-form values in the E4M3 definition
  (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals
  k * 2^-9, largest finite 448, S.1111.111 is NaN).
* Encoding by brute force: for random and hand-picked fp32 inputs, the code is
  the finite E4M3 value nearest the input in exact arithmetic, ties to the
  even mantissa, saturating at +-448 -- found by scanning all 254 finite codes.
* The group quantiser: scale = amax/448 rounded, largest code +-448 in every
  group with a normal scale, signs, monotonicity, and a dequantisation error
  within half an E4M3 step of the scaled value.
* The whole pass: composition of the (pinned) intermediates with the FP8 group
  quantiser along both axes, and an fp64 error bound of the dequantised values.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from exact import rn32
from swiglu_backward_int8_amd.inputs import make_inputs, random_inputs

G = 128
FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


def _value(c):
    s = -1 if c & 0x80 else 1
    e, m = (c >> 3) & 0xF, c & 7
    if e == 0:
        return s * Fraction(m, 512)
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def test_decode_closed_forms():
    assert oracle.e4m3_to_float(0x38) == 1.0
    assert oracle.e4m3_to_float(0x7E) == 448.0 and oracle.e4m3_to_float(0xFE) == -448.0
    assert oracle.e4m3_to_float(0x01) == 2.0**-9 and oracle.e4m3_to_float(0x07) == 7 * 2.0**-9
    assert oracle.e4m3_to_float(0x08) == 2.0**-6
    assert oracle.e4m3_to_float(0x40) == 2.0 and oracle.e4m3_to_float(0x3C) == 1.5
    assert np.isnan(oracle.e4m3_to_float(0x7F)) and np.isnan(oracle.e4m3_to_float(0xFF))
    for c in FINITE:
        assert Fraction(oracle.e4m3_to_float(c)) == _value(c)


def _nearest(x: Fraction) -> int:
    if x == 0:
        return 0
    best = None
    for c in FINITE:
        if (c & 0x80) != (0x80 if x < 0 else 0):
            continue
        d = abs(_value(c) - x)
        key = (d, c & 1)  # ties: even mantissa (lowest bit of the code)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_encode_brute_force():
    rng = np.random.default_rng(31)
    xs = list(rng.standard_normal(600) * 10.0 ** rng.uniform(-4, 2.7, 600))
    # midpoints, boundary values, saturation
    for c in range(0x00, 0x7E):
        a, b = _value(c), _value(c + 1)
        xs += [float((a + b) / 2), float(a), -float((a + b) / 2)]
    xs += [448.0, 460.0, 464.0, 1000.0, -1e30, 2.0**-10, 3 * 2.0**-11, 1e-30]
    for x in xs:
        x32 = float(np.float32(x))
        got = oracle.f32_to_e4m3(x32)
        X = Fraction(x32)
        if abs(X) >= 448:
            want = 0xFE if X < 0 else 0x7E
        else:
            want = _nearest(X)
        if X == 0:
            assert _value(got) == 0
            continue
        assert got == want, (x32, hex(got), hex(want))


def test_signed_zero_and_saturation():
    # E4M3 has a negative zero (0x80); the encoder keeps the sign of a zero
    # input, and a zero value quantises to the zero of its own sign, also in a
    # group whose inverse scale overflows (where 0 * inf would be NaN).
    assert oracle.f32_to_e4m3(0.0) == 0x00 and oracle.f32_to_e4m3(-0.0) == 0x80
    q, s = oracle.quant_group_fp8([-0.0, 1.0, 0.0])
    assert q.tolist() == [0x80, 0x7E, 0x00] and Fraction(float(s)) == rn32(Fraction(1, 448))
    # amax = 2^-130: scale = 2^-130 / 448 is subnormal and 1/scale is inf, so
    # every non-zero value saturates to +-448
    tiny = 2.0**-130
    q, s = oracle.quant_group_fp8([tiny, -tiny / 2, 0.0, tiny / 8, -0.0])
    assert q.tolist() == [0x7E, 0xFE, 0x00, 0x7E, 0x80]
    assert Fraction(float(s)) == rn32(Fraction(tiny) / 448) and np.isinf(np.float32(1) / s)
    # an all-zero group has scale 1.0 (not 0), so dequantisation stays finite
    q, s = oracle.quant_group_fp8([0.0] * 128)
    assert s == 1.0 and not q.any()
    q, s = oracle.quant_group_fp8([-0.0, 0.0, -0.0])
    assert s == 1.0 and q.tolist() == [0x80, 0x00, 0x80]
    # magnitudes beyond the largest finite value saturate; none becomes NaN
    for x, c in ((448.0, 0x7E), (463.9, 0x7E), (464.0, 0x7E), (1e38, 0x7E), (-3e5, 0xFE)):
        assert oracle.f32_to_e4m3(x) == c


def test_group_quantiser_invariants():
    rng = np.random.default_rng(32)
    for i in range(300):
        n = int(rng.integers(1, 129))
        v = (rng.standard_normal(n) * 10.0 ** rng.uniform(-20, 20)).astype(np.float32)
        v = np.array([oracle.bf16_to_f32(oracle.f32_to_bf16(float(a))) for a in v], np.float32)
        if i % 9 == 0:
            v[: n // 3] = 0.0
        q, s = oracle.quant_group_fp8(v)
        amax = float(np.max(np.abs(v)))
        if amax == 0.0:
            assert s == 1.0 and not q.any()
            continue
        assert Fraction(float(s)) == rn32(Fraction(amax) / 448)
        vals = np.array([oracle.e4m3_to_float(c) for c in q])
        if float(s) >= 2.0**-126:
            assert np.max(np.abs(vals)) == 448.0
        assert np.all((vals == 0) | (np.sign(vals) == np.sign(v)))
        order = np.argsort(v, kind="stable")
        assert np.all(np.diff(vals[order]) >= 0)
        t = np.abs(v.astype(np.float64) / float(s))
        step = np.where(t >= 2.0**-6, 2.0 ** (np.floor(np.log2(np.maximum(t, 2.0**-6))) - 3), 2.0**-9)
        err = np.abs(vals * float(s) - v.astype(np.float64))
        assert np.all(err <= float(s) * step * (0.5 + 2.0**-10) + 1e-300)


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("T,H", [(256, 256), (200, 384)])
def test_pass_is_composition(T, H):
    x, dy = random_inputs(T, H, seed=T + H)
    xb, db = _bits(x), _bits(dy)
    gq, gs, yq, ys = oracle.silu_dot_fwd_bwd_quant_fuse_fp8(xb, db)
    Y, D = oracle.intermediates(xb, db)
    for t in range(0, T, 23):
        for j in range(-(-2 * H // G)):
            q, s = oracle.quant_group_fp8(D[t, j * G:(j + 1) * G])
            assert np.array_equal(q, gq[t, j * G:(j + 1) * G]) and s == gs[t, j]
    for h in range(0, H, 29):
        for j in range(-(-T // G)):
            q, s = oracle.quant_group_fp8(Y[j * G:(j + 1) * G, h])
            assert np.array_equal(q, yq[h, j * G:(j + 1) * G]) and s == ys[h, j]


def test_pass_fp64_error_bound():
    x, dy = make_inputs("t32768_h2048_outliers", device="cpu", T=256)
    H = dy.shape[1]
    xs = torch.cat([x[:, :256], x[:, H:H + 256]], dim=1).contiguous()
    ds = dy[:, :256].contiguous()
    xb, db = _bits(xs), _bits(ds)
    gq, gs, yq, ys = oracle.silu_dot_fwd_bwd_quant_fuse_fp8(xb, db)
    xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    df = (db.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    g, u = xf[:, :256], xf[:, 256:]
    with np.errstate(over="ignore"):
        s = 1 / (1 + np.exp(-g))
    y = g * s * u
    dec = np.vectorize(oracle.e4m3_to_float)
    deq = dec(yq) * np.repeat(ys.astype(np.float64), G, axis=1)[:, :256]
    # e4m3 keeps 4 significant bits: relative rounding <= 2^-4, plus bf16 2^-8
    sc = np.repeat(ys.astype(np.float64), G, axis=1)[:, :256]
    assert np.all(np.abs(deq - y.T) <= np.abs(y.T) * (2.0**-4 + 2.0**-8 + 2.0**-12) + sc * 2.0**-9)
