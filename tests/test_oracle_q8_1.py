"""Pins for the binary16 encoder and the q8_1 block layout of the oracle (CPU).

* oracle_f32_to_f16 against numpy's float32 -> float16 conversion (IEEE
  round to nearest, ties to even): random finite patterns, every midpoint
  between neighbouring binary16 values (ties), the subnormal and overflow
  edges, signed zeros and infinities.
* oracle_silu_fwd_quant_q8_1: a saturated-gate block in closed form (every
  code 127, d and sum from the exact scale), and on random rows the layout
  taken apart with numpy: the codes are the group-32 forward quantiser's, d is
  its scale in binary16 and the sum is fl32(scale * sum(q)) in binary16, both
  converted by numpy; the sum stays within the codes' rounding of the block's
  own y values.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from exact import rn32
from swiglu_backward_int8_amd.inputs import random_inputs


def _np_f16_bits(a):
    return np.asarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def _oracle_f16_bits(a):
    return np.array([oracle.f32_to_f16(float(v)) for v in np.asarray(a, dtype=np.float32).ravel()], dtype=np.uint16)


def test_f16_random_patterns():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, 120_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    # keep most of them within and near binary16's range
    near = (rng.random(40_000) * 2 - 1).astype(np.float32) * np.float32(2.0) ** rng.integers(-30, 18, 40_000).astype(np.float32)
    v = np.concatenate([v[:60_000], near])
    with np.errstate(over="ignore"):
        assert np.array_equal(_oracle_f16_bits(v), _np_f16_bits(v))


def test_f16_every_midpoint_ties_to_even():
    h = np.arange(0, 0x7C00, dtype=np.uint16)  # every finite non-negative binary16
    lo = h[:-1].view(np.float16).astype(np.float64)
    hi = h[1:].view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)  # exact: 12 significant bits
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    got = _oracle_f16_bits(np.concatenate([mid, -mid]))
    want = np.concatenate([np.where(h[:-1] % 2 == 0, h[:-1], h[1:]), np.where(h[:-1] % 2 == 0, h[:-1], h[1:]) | 0x8000])
    assert np.array_equal(got, want.astype(np.uint16))


def test_f16_edges():
    cases = [(65504.0, 0x7BFF), (65519.996, 0x7BFF), (65520.0, 0x7C00), (1e9, 0x7C00), (float("inf"), 0x7C00),
             (-float("inf"), 0xFC00), (0.0, 0x0000), (-0.0, 0x8000), (2.0**-24, 0x0001), (2.0**-25, 0x0000),
             (3 * 2.0**-25, 0x0002), (2.0**-14, 0x0400), (2.0**-14 - 2.0**-24, 0x03FF), (1.0, 0x3C00),
             (-2.5, 0xC100), (1e-30, 0x0000)]
    for x, want in cases:
        assert oracle.f32_to_f16(x) == want, (x, hex(oracle.f32_to_f16(x)))


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_q8_1_saturated_block_closed_form():
    # gate 20 (s == 1), up 1: y = 20 exactly in every channel, so each block
    # has scale rn(20/127), all codes 127, sum(q) = 32 * 127
    T, H = 3, 64
    x = torch.empty((T, 2 * H), dtype=torch.bfloat16)
    x[:, :H] = 20.0
    x[:, H:] = 1.0
    out = oracle.silu_fwd_quant_q8_1(_bits(x))
    assert out.shape == (T, 2 * 36)
    d, s, q = oracle.split_q8_1(out)
    scale = rn32(Fraction(20) / 127)
    total = rn32(Fraction(float(scale)) * 4064)
    assert np.all(q == 127)
    assert np.all(d == np.float16(np.float32(float(scale))))
    assert np.all(s == np.float16(np.float32(float(total))))
    # byte order: d's low byte first, then sum, then the codes
    dbits = int(np.float16(np.float32(float(scale))).view(np.uint16))
    assert out[0, 0] == dbits & 0xFF and out[0, 1] == dbits >> 8 and out[0, 4] == 127


@pytest.mark.parametrize("T,H,weighted", [(16, 256, False), (9, 96, True), (5, 32, False)])
def test_q8_1_layout_against_the_forward_quantiser(T, H, weighted):
    xt, _ = random_inputs(T, H, seed=T + H)
    xb = _bits(xt)
    w = (np.random.default_rng(T).random(T) * 4 - 2).astype(np.float32) if weighted else None
    out = oracle.silu_fwd_quant_q8_1(xb, w)
    d, s, q = oracle.split_q8_1(out)
    yq, ys, yb = oracle.silu_fwd_quant(xb, w, group_size=32, want_bf16=True)
    assert np.array_equal(q.reshape(T, H), yq)
    assert np.array_equal(d.view(np.uint16), _np_f16_bits(ys))
    qsum = yq.reshape(T, -1, 32).astype(np.int32).sum(axis=2)
    assert np.array_equal(s.view(np.uint16), _np_f16_bits(ys * qsum.astype(np.float32)))
    # the sum is the block's values as the codes give them: within half a
    # step per code (plus the binary16 rounding) of the sum of y itself
    y = (yb.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(T, -1, 32).sum(axis=2)
    bound = 16 * ys.astype(np.float64) * (1 + 2.0**-14) + np.abs(y) * 2.0**-10 + 1e-7
    assert np.all(np.abs(s.astype(np.float64) - y) <= bound)


def test_q8_1_needs_h_a_multiple_of_32():
    xt, _ = random_inputs(4, 48, seed=3)
    with pytest.raises(RuntimeError):
        oracle.silu_fwd_quant_q8_1(_bits(xt))


# The page's own argument shape (kquant_swiglu_q8_1_rows on the page
# "kquant_mmq.rs"): separate gate and up arrays, an optional row weight, and
# both the bf16 h and its q8_1 blocks written.  The page states the fused
# launch is byte-identical to the swiglu launch followed by the q8_1 launch;
# here that is the pinned forward quantiser (for h) and the pinned q8_1
# layout (for the blocks) on x = [gate | up].

@pytest.mark.parametrize("rows,inter,weighted", [(16, 256, False), (9, 96, True), (5, 32, True), (1, 64, False)])
def test_separate_gate_up_equals_the_two_launches(rows, inter, weighted):
    xt, _ = random_inputs(rows, inter, seed=3 * rows + inter)
    xb = _bits(xt)
    gate = np.ascontiguousarray(xb[:, :inter])
    up = np.ascontiguousarray(xb[:, inter:])
    w = (np.random.default_rng(rows).random(rows) * 4 - 2).astype(np.float32) if weighted else None
    blocks, h = oracle.kquant_swiglu_q8_1_rows(gate, up, w)
    _, _, yb = oracle.silu_fwd_quant(xb, w, group_size=32, want_bf16=True)
    assert np.array_equal(h, yb)
    assert np.array_equal(blocks, oracle.silu_fwd_quant_q8_1(xb, w))
    assert np.array_equal(oracle.kquant_swiglu_q8_1_rows(gate, up, w, want_h=False), blocks)


def test_separate_gate_up_saturated_closed_form():
    # gate 20 (s == 1), up 0.5, weight 3: h = bf16(10 * 3) = 30 exactly in
    # every channel; scale rn(30/127), codes 127, sum(q) = 32 * 127
    rows, inter = 2, 64
    gate = np.full((rows, inter), 0x41A0, dtype=np.uint16)  # bf16 20.0
    up = np.full((rows, inter), 0x3F00, dtype=np.uint16)    # bf16 0.5
    blocks, h = oracle.kquant_swiglu_q8_1_rows(gate, up, np.full(rows, 3.0, dtype=np.float32))
    assert np.all(h == 0x41F0)  # bf16 30.0
    d, s, q = oracle.split_q8_1(blocks)
    scale = rn32(Fraction(30) / 127)
    assert np.all(q == 127)
    assert np.all(d == np.float16(np.float32(float(scale))))
    assert np.all(s == np.float16(np.float32(float(rn32(Fraction(float(scale)) * 4064)))))


def test_separate_gate_up_needs_inter_a_multiple_of_32():
    g = np.zeros((2, 48), dtype=np.uint16)
    with pytest.raises(RuntimeError):
        oracle.kquant_swiglu_q8_1_rows(g, g)
