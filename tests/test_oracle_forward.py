"""Pins for the oracle's forward quantiser (CPU only).

oracle_silu_fwd_quant computes y = bf16((silu(g) * u) * w[t]) and quantises
each row in groups of 128 channels.  Pinned by:

* composition: it equals the backward pass's own bf16 y (pinned elsewhere)
  quantised row by row with the pinned group quantiser -- the fused launch is
  the composition of the two steps;
* the weight: w = 1 and no weight agree bit for bit; w = 2 (a power of two)
  doubles every bf16 value exactly, leaves every code alone and doubles every
  scale; w = -1 negates every code; w = 0 gives zero codes and scale 1.0;
* an fp64 error bound of the dequantised values against the exact
  silu(g) * u * w;
* a trailing partial group (H not a multiple of 128) quantised over its own
  elements.
"""

import numpy as np
import pytest
import torch

import oracle
from swiglu_backward_int8_amd.inputs import make_inputs, random_inputs

G = 128


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("name", ["t256_h256", "t8192_h4096", "t32768_h2048_outliers"])
def test_composition_with_backward_y(name):
    x, dy = make_inputs(name, device="cpu", T=256)
    H = dy.shape[1]
    xb, db = _bits(x), _bits(dy)
    yq, ys, yb = oracle.silu_fwd_quant(xb, want_bf16=True)
    Y, _ = oracle.intermediates(xb, db)
    assert np.array_equal((yb.astype(np.uint32) << 16).view(np.float32), Y)
    for t in range(0, 256, 37):
        for j in range(H // G):
            q, s = oracle.quant_group(Y[t, j * G:(j + 1) * G])
            assert np.array_equal(q, yq[t, j * G:(j + 1) * G]) and s == ys[t, j]


def test_row_weights():
    x, _ = random_inputs(128, 256, seed=21)
    xb = _bits(x)
    base = oracle.silu_fwd_quant(xb, want_bf16=True)
    one = oracle.silu_fwd_quant(xb, w=np.ones(128, np.float32), want_bf16=True)
    assert all(np.array_equal(a, b) for a, b in zip(base, one))
    two = oracle.silu_fwd_quant(xb, w=np.full(128, 2.0, np.float32), want_bf16=True)
    yb1 = (base[2].astype(np.uint32) << 16).view(np.float32)
    yb2 = (two[2].astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(yb2, 2 * yb1)
    assert np.array_equal(two[0], base[0]) and np.array_equal(two[1], 2 * base[1])
    neg = oracle.silu_fwd_quant(xb, w=np.full(128, -1.0, np.float32))
    assert np.array_equal(neg[0], -base[0]) and np.array_equal(neg[1], base[1])
    zero = oracle.silu_fwd_quant(xb, w=np.zeros(128, np.float32))
    assert not zero[0].any() and np.all(zero[1] == 1.0)


def test_fp64_error_bound_with_weights():
    x, _ = random_inputs(256, 384, seed=22, gate_std=2.0)
    xb = _bits(x)
    w = np.random.default_rng(3).uniform(-2, 2, 256).astype(np.float32)
    yq, ys = oracle.silu_fwd_quant(xb, w=w)
    xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    g, u = xf[:, :384], xf[:, 384:]
    exact = g / (1 + np.exp(-g)) * u * w[:, None].astype(np.float64)
    sc = np.repeat(ys.astype(np.float64), G, axis=1)
    err = np.abs(yq * sc - exact)
    assert np.all(err <= sc * (0.5 + 2.0**-15) + np.abs(exact) * (2.0**-8 + 2.0**-20))


def test_partial_trailing_group():
    x, _ = random_inputs(64, 200, seed=23)
    xb = _bits(x)
    yq, ys, yb = oracle.silu_fwd_quant(xb, want_bf16=True)
    assert ys.shape == (64, 2)
    Y = (yb.astype(np.uint32) << 16).view(np.float32)
    for t in range(64):
        q, s = oracle.quant_group(Y[t, 128:])
        assert np.array_equal(q, yq[t, 128:]) and s == ys[t, 1]
