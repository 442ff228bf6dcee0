"""Parity of the forward quantiser (silu_fwd_quant) with the CPU oracle (GPU).

Same bar as the backward pass: scales within 1e-6 relative, codes equal except
|dq| <= 1 on at most 1e-4 of them; the cases assert exact equality, which holds.
"""

import numpy as np
import pytest
import torch

import oracle
import swiglu_backward_int8_amd as sq
from swiglu_backward_int8_amd.inputs import WORKLOADS, make_inputs, random_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run(x, w=None, want_bf16=False, group=128):
    T, H = x.shape[0], x.shape[1] // 2
    yq = torch.full((T, H), -7, dtype=torch.int8, device=DEV)
    ys = torch.full((T, -(-H // group)), float("nan"), dtype=torch.float32, device=DEV)
    yb = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=DEV) if want_bf16 else None
    sq.silu_fwd_quant(x, yq, ys, row_weight=w, y_bf16=yb, group_size=group)
    torch.cuda.synchronize()
    out = [yq.cpu().numpy(), ys.cpu().numpy()]
    if want_bf16:
        out.append(_bits(yb))
    return out


def check(x, w=None, want_bf16=False, label="", group=128):
    got = run(x, w, want_bf16, group)
    want = oracle.silu_fwd_quant(_bits(x), None if w is None else w.cpu().numpy(), group_size=group,
                                 want_bf16=want_bf16)
    assert np.array_equal(got[1].view(np.uint32), want[1].view(np.uint32)), "%s: scales differ" % label
    d = np.abs(got[0].astype(np.int16) - want[0].astype(np.int16))
    assert int(d.max(initial=0)) == 0, "%s: %d codes differ" % (label, int((d > 0).sum()))
    if want_bf16:
        assert np.array_equal(got[2], want[2]), "%s: bf16 y differs" % label
    print("%s exact" % label, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available()
    sq.prepare()


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workloads(name):
    # every workload at its full token count
    print("case forward", name, flush=True)
    x, _ = make_inputs(name, device=DEV)
    check(x, want_bf16=True, label=name)


@pytest.mark.parametrize("name", ["t4096_h1408", "t32768_h2048_outliers"])
def test_row_weights(name):
    x, _ = make_inputs(name, device=DEV, T=2048)
    gen = torch.Generator(device=DEV).manual_seed(5)
    w = (torch.rand(x.shape[0], generator=gen, device=DEV) * 4 - 2).contiguous()
    w[::17] = 0.0
    check(x, w=w, want_bf16=True, label=name + " weighted")


@pytest.mark.parametrize("T", [1, 3, 5, 127, 1000, 4097])
def test_ragged_token_counts(T):
    x, _ = random_inputs(T, 384, device=DEV, seed=T)
    check(x, want_bf16=(T % 2 == 1), label="T=%d" % T)


def test_without_bf16_output_matches():
    x, _ = random_inputs(512, 256, device=DEV, seed=9)
    a = run(x, want_bf16=False)
    b = run(x, want_bf16=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_edge_values():
    T, H = 64, 256
    x = torch.zeros((T, 2 * H), dtype=torch.bfloat16, device=DEV)
    x[:, :H] = torch.linspace(-100, 30, H, device=DEV).to(torch.bfloat16)
    x[:, H:] = 1.0
    x[1, :] = 0.0  # all-zero row: scale 1.0, codes 0
    x[2, H:] = 2.0**-130  # tiny groups: inverse overflows
    x[2, :H] = 20.0
    check(x, want_bf16=True, label="edges")


def test_empty_and_errors():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    sq.silu_fwd_quant(x, torch.empty((0, 128), dtype=torch.int8, device=DEV),
                      torch.empty((0, 1), dtype=torch.float32, device=DEV))
    x, _ = random_inputs(8, 200, device=DEV)
    with pytest.raises(ValueError):  # y_s must be [8, ceil(200 / 128)]
        sq.silu_fwd_quant(x, torch.empty((8, 200), dtype=torch.int8, device=DEV),
                          torch.empty((8, 1), dtype=torch.float32, device=DEV))
    x, _ = random_inputs(8, 100, device=DEV)
    with pytest.raises(ValueError):  # y_q must be [8, 100]
        sq.silu_fwd_quant(x, torch.empty((8, 104), dtype=torch.int8, device=DEV),
                          torch.empty((8, 1), dtype=torch.float32, device=DEV))


def test_forward_y_equals_backward_recompute():
    # without a row weight the forward y is the y the backward pass quantises
    x, dy = make_inputs("t4096_h1408", device=DEV, T=512)
    yb = run(x, want_bf16=True)[2]
    y, _ = sq.eval_intermediates(x, dy)
    assert np.array_equal(yb, _bits(y))


# Groups of 64 and 32 channels, and H any multiple of the group (the last
# 128-channel block then holds 32, 64 or 96 channels).
@pytest.mark.parametrize("T,H,group", [(256, 256, 64), (256, 256, 32), (301, 192, 64), (1000, 160, 32),
                                       (5, 96, 32), (4096, 1376, 32), (4099, 448, 64), (1, 64, 64)])
def test_forward_groups_and_ragged_h(T, H, group):
    x, _ = random_inputs(T, H, device=DEV, seed=7 * T + H + group)
    w = torch.rand(T, device=DEV, generator=torch.Generator(device=DEV).manual_seed(T)) * 4 - 2
    check(x, label="T=%d H=%d group=%d" % (T, H, group), group=group)
    check(x, w=w, want_bf16=True, label="T=%d H=%d group=%d weighted" % (T, H, group), group=group)


# H any multiple of 8: the last group of a row is partial, and with
# H % 16 == 8 each lane stores its own 8 codes.
@pytest.mark.parametrize("T,H,group", [(100, 200, 128), (64, 40, 32), (300, 1000, 64), (17, 8, 128),
                                       (1000, 1064, 128), (129, 2056, 32), (5, 24, 64)])
def test_forward_partial_groups(T, H, group):
    x, _ = random_inputs(T, H, device=DEV, seed=3 * T + H + group)
    w = torch.rand(T, device=DEV, generator=torch.Generator(device=DEV).manual_seed(T)) * 4 - 2
    check(x, label="T=%d H=%d group=%d" % (T, H, group), group=group)
    check(x, w=w, want_bf16=True, label="T=%d H=%d group=%d weighted" % (T, H, group), group=group)


@pytest.mark.parametrize("group", [32, 64])
def test_forward_groups_workload(group):
    x, _ = make_inputs("t32768_h2048_outliers", device=DEV)
    check(x, label="outliers group=%d" % group, group=group)


# H not a multiple of 8: rows off 16 bytes, so the tiled kernel loads aligned
# pieces and shifts them across lanes, and stores y_q and y_bf16 as aligned
# pieces with only the unit's own bytes at both ends of a row (rows of 4
# tokens start at every offset class; T ragged at 4).
@pytest.mark.parametrize("T,H,group", [(100, 100, 128), (64, 5, 32), (300, 1001, 64), (17, 1, 128), (129, 2050, 32),
                                       (9, 129, 128), (7, 255, 64), (31, 4095, 32), (2048, 11001, 128),
                                       (65, 11003, 64), (3, 127, 32)])
def test_forward_h_not_a_multiple_of_8(T, H, group):
    x, _ = random_inputs(T, H, device=DEV, seed=5 * T + H + group)
    w = torch.rand(T, device=DEV, generator=torch.Generator(device=DEV).manual_seed(T)) * 4 - 2
    check(x, label="narrow T=%d H=%d group=%d" % (T, H, group), group=group)
    check(x, w=w, want_bf16=True, label="narrow T=%d H=%d group=%d weighted" % (T, H, group), group=group)


def _random_narrow_shapes(n=10, seed=9091):
    rng = np.random.default_rng(seed)
    shapes = []
    for i in range(n):
        H = int(rng.integers(1, 3000))
        if H % 8 == 0:
            H += int(rng.integers(1, 8))
        shapes.append((int(rng.integers(1, 700)), H, int(rng.choice([32, 64, 128]))))
    return shapes


@pytest.mark.parametrize("T,H,group", _random_narrow_shapes())
def test_forward_h_not_a_multiple_of_8_random(T, H, group):
    x, _ = random_inputs(T, H, device=DEV, seed=11 * T + H)
    w = torch.rand(T, device=DEV, generator=torch.Generator(device=DEV).manual_seed(H)) * 4 - 2
    check(x, w=w, want_bf16=True, label="narrow random T=%d H=%d group=%d weighted" % (T, H, group), group=group)


def _takes_wide_rows(H):
    # the library's choice for H not a multiple of 8: rows of 512-channel units
    # when H >= 1024 and they pad a row by at most 3% more than 128-channel units
    wide, narrow = -(-H // 512) * 512, -(-H // 128) * 128
    return H % 8 != 0 and H >= 1024 and 100 * wide <= 103 * narrow


# Long rows take units of one token x 512 channels, each unit's codes and y
# stored as one run of aligned pieces: rows that fill their units, a last unit
# of 511 channels or of one channel, every offset class of a row's start.
@pytest.mark.parametrize("T,H,group", [(5, 1535, 128), (9, 2047, 64), (3, 4607, 32), (5, 33281, 128), (130, 3583, 128),
                                       (66, 6143, 64), (7, 1531, 32), (17, 12287, 128)])
def test_forward_wide_rows(T, H, group):
    assert _takes_wide_rows(H)
    x, _ = random_inputs(T, H, device=DEV, seed=7 * T + H + group)
    w = torch.rand(T, device=DEV, generator=torch.Generator(device=DEV).manual_seed(H + 1)) * 4 - 2
    check(x, label="wide rows T=%d H=%d group=%d" % (T, H, group), group=group)
    check(x, w=w, want_bf16=True, label="wide rows T=%d H=%d group=%d weighted" % (T, H, group), group=group)


@pytest.mark.parametrize("group", [128, 64, 32])
def test_forward_tiny_group_maxima_wide_rows(group):
    # as below, with H = 1535 (units of 512 channels): the clamped rule there
    T, H = 40, 1535
    assert _takes_wide_rows(H)
    t = torch.arange(T, dtype=torch.float64).unsqueeze(1)
    j = torch.arange(H, dtype=torch.float64).unsqueeze(0)
    up = ((1 + (j % 64) / 64) * torch.pow(2.0, -110 - t)).to(torch.float32)
    x = torch.cat([torch.full((T, H), 20.0), up], dim=1).to(torch.bfloat16).to(DEV)
    check(x, label="tiny maxima H=1535 group=%d" % group, group=group)
    w = torch.full((T,), 0.75, dtype=torch.float32, device=DEV)
    check(x, w=w, want_bf16=True, label="tiny maxima H=1535 weighted group=%d" % group, group=group)


@pytest.mark.parametrize("group", [128, 64, 32])
def test_forward_tiny_group_maxima_h_not_a_multiple_of_8(group):
    # as below, with H = 251: the clamped rule on the shifted path
    T, H = 40, 251
    t = torch.arange(T, dtype=torch.float64).unsqueeze(1)
    j = torch.arange(H, dtype=torch.float64).unsqueeze(0)
    up = ((1 + (j % 64) / 64) * torch.pow(2.0, -110 - t)).to(torch.float32)
    x = torch.cat([torch.full((T, H), 20.0), up], dim=1).to(torch.bfloat16).to(DEV)
    check(x, label="tiny maxima H=251 group=%d" % group, group=group)
    w = torch.full((T,), 0.75, dtype=torch.float32, device=DEV)
    check(x, w=w, want_bf16=True, label="tiny maxima H=251 weighted group=%d" % group, group=group)


@pytest.mark.parametrize("group", [128, 64, 32])
def test_forward_tiny_group_maxima(group):
    # gate 20 (sigmoid exactly 1) and up = (1 + j/64) * 2^(-110 - t): row t's
    # group maxima run from 2^-106 down through 2^-119 (below which the kernel
    # leaves its scale table for the divisions), the overflowing inverses
    # (amax < 127 * 2^-128) and subnormal y, to zero rows
    T, H = 40, 256
    t = torch.arange(T, dtype=torch.float64).unsqueeze(1)
    j = torch.arange(H, dtype=torch.float64).unsqueeze(0)
    up = ((1 + (j % 64) / 64) * torch.pow(2.0, -110 - t)).to(torch.float32)
    x = torch.cat([torch.full((T, H), 20.0), up], dim=1).to(torch.bfloat16).to(DEV)
    check(x, label="tiny maxima group=%d" % group, group=group)
    w = torch.full((T,), 0.75, dtype=torch.float32, device=DEV)
    check(x, w=w, want_bf16=True, label="tiny maxima weighted group=%d" % group, group=group)
    q8 = torch.empty((T, H // 32 * sq.Q8_1_BLOCK), dtype=torch.uint8, device=DEV)
    if group == 32:
        sq.silu_fwd_quant_q8_1(x, q8)
        torch.cuda.synchronize()
        assert np.array_equal(q8.cpu().numpy(), oracle.silu_fwd_quant_q8_1(_bits(x)))
