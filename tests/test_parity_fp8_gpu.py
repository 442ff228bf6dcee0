"""Parity of the FP8 (OCP E4M3) variant of the pass with the CPU oracle (GPU).

The kernel reproduces the oracle's arithmetic operation for operation (the same
bf16 intermediates, scale = amax / 448 by fp32 division, the fp32 product
v * inv, one round-to-nearest-even conversion), so the bar is bit equality of
every code byte and every scale.  Besides the oracle comparison the cases check
properties that hold at any size: no NaN code (0x7F, 0xFF) is ever written,
and every group with a normal-range scale holds a code of magnitude 448.
"""

import numpy as np
import pytest
import torch

import oracle
import swiglu_backward_int8_amd as sq
from swiglu_backward_int8_amd.inputs import WORKLOADS, make_inputs, random_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAMES = ("grad_input_q", "grad_input_s", "y_q_t", "y_s_t")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sq.lib()
    sq.prepare()


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_gpu(x, grad_y):
    T, H = grad_y.shape
    outs = sq.empty_outputs(T, H, x.device, fp8=True)
    for o in outs:  # poison: every element must be written (0x7F is a NaN code)
        o.fill_(0x7F if o.dtype == torch.uint8 else float("nan"))
    sq.silu_dot_fwd_bwd_quant_fuse_fp8(x, grad_y, *outs)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


def compare(got, want, label=""):
    report = {}
    for name, g, w in zip(NAMES, got, want):
        assert g.shape == w.shape, (name, g.shape, w.shape)
        if g.dtype == np.float32:
            bad = np.nonzero(g.view(np.uint32) != w.view(np.uint32))
        else:
            assert not np.isin(g, (0x7F, 0xFF)).any(), "%s %s: NaN code written" % (label, name)
            bad = np.nonzero(g != w)
        report[name] = int(bad[0].size)
        assert bad[0].size == 0, "%s %s: %d differ, first at %s: got %r want %r" % (
            label, name, bad[0].size, tuple(int(b[0]) for b in bad), g[tuple(b[0] for b in bad)],
            w[tuple(b[0] for b in bad)])
    print("%s mismatches %s" % (label, report), flush=True)
    return report


def check(x, grad_y, label):
    got = run_gpu(x, grad_y)
    want = oracle.silu_dot_fwd_bwd_quant_fuse_fp8(_bits(x), _bits(grad_y))
    compare(got, want, label)
    return got


def _full_scale_codes_present(q: np.ndarray, s: np.ndarray, axis: int):
    """Every group whose scale is a normal fp32 number holds a code of magnitude
    448 (0x7E or 0xFE): its largest value times the inverse scale rounds to 448."""
    mag = (q & 0x7F) == 0x7E
    if axis == 1:  # grad_input_q rows: groups of 128 contiguous codes
        T, W = q.shape
        has = mag.reshape(T, W // 128, 128).any(axis=2)
    else:  # y_q_t rows: groups of 128 consecutive tokens, the last one shorter
        H, T = q.shape
        pad = (-T) % 128
        has = np.pad(mag, ((0, 0), (0, pad))).reshape(H, -1, 128).any(axis=2)
    normal = np.abs(s) >= np.float32(2.0**-126)
    amax_zero = s == 1.0  # an all-zero group has scale 1 and only zero codes
    assert np.all(has | ~normal | amax_zero)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_parity_fp8(name):
    print("case fp8", name, flush=True)
    x, dy = make_inputs(name, device=DEV)
    got = check(x, dy, "fp8 " + name)
    _full_scale_codes_present(got[0], got[1], axis=1)
    _full_scale_codes_present(got[2], got[3], axis=0)


@pytest.mark.parametrize("name,seed", [("t4096_h1408", 2001), ("t32768_h2048_outliers", 2004)])
def test_workload_parity_fp8_second_seed(name, seed):
    print("case fp8", name, seed, flush=True)
    x, dy = make_inputs(name, device=DEV, seed=seed)
    check(x, dy, "fp8 %s seed %d" % (name, seed))


@pytest.mark.parametrize("T,H", [(1, 128), (100, 256), (129, 128), (200, 384), (1023, 128), (4097, 384),
                                 (333, 1408)])
def test_ragged_token_counts_fp8(T, H):
    x, dy = random_inputs(T, H, device=DEV, seed=T * 11 + H)
    check(x, dy, "fp8 ragged T=%d H=%d" % (T, H))


def _const(T, H, g, u, d):
    x = torch.empty((T, 2 * H), dtype=torch.bfloat16, device=DEV)
    x[:, :H] = g
    x[:, H:] = u
    return x, torch.full((T, H), d, dtype=torch.bfloat16, device=DEV)


def test_rounding_ties_and_subnormal_codes():
    # gate = 100: s == 1 exactly, so d_gate == grad_y * up exactly; with
    # grad_y = 1 and 448 in the group the scale and its inverse are exactly 1
    # and each code is the E4M3 rounding of the up value itself.
    T = H = 128
    x, dy = _const(T, H, 100.0, 0.0, 1.0)
    vals = [448.0, 1.0625, 1.1875, -1.0625, 2.0**-10, 3 * 2.0**-10, 15 * 2.0**-10, -0.0, 0.0, 240.0]
    x[:, H:H + len(vals)] = torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).to(DEV)
    got = check(x, dy, "fp8 ties")
    # 448 -> 0x7E; 1 + 1/16 is halfway between 1 and 1.125 -> 1 (0x38, even);
    # 1 + 3/16 is halfway between 1.125 and 1.25 -> 1.25 (0x3A, even); the
    # negative tie -> 0xB8; 2^-10 is half the smallest subnormal 2^-9 -> 0;
    # 1.5 * 2^-9 -> 2 * 2^-9 (0x02); 7.5 * 2^-9 -> 2^-6, the smallest normal
    # (0x08); -0 keeps its sign (0x80); 240 = 1.875 * 2^7 -> 0x77.
    assert got[0][0, :len(vals)].tolist() == [0x7E, 0x38, 0x3A, 0xB8, 0x00, 0x02, 0x08, 0x80, 0x00, 0x77]
    assert got[1][0, 0] == 1.0


def test_tiny_groups_overflowing_inverse_fp8():
    # group maximum 2^-130: scale = 2^-130 / 448 is a subnormal fp32 number and
    # 1/scale overflows to inf; non-zero values saturate to +-448, zeros keep
    # their sign.
    T = H = 128
    x, dy = _const(T, H, 20.0, 0.0, 1.0)
    tiny = torch.tensor([2.0**-130, -(2.0**-131), 0.0, 2.0**-133, -0.0], dtype=torch.float32)
    x[:, H:H + 5] = tiny.to(torch.bfloat16).to(DEV)
    got = check(x, dy, "fp8 tiny groups")
    assert got[0][0, :5].tolist() == [0x7E, 0xFE, 0x00, 0x7E, 0x80]


@pytest.mark.parametrize("g,u,d", [(0.0, 1.0, 1.0), (1.0, -1.0, 1.0), (-100.0, 1.0, 1.0), (0.0, 0.0, 0.0),
                                   (3.0, -0.0, 1.0)])
def test_constant_inputs_fp8(g, u, d):
    x, dy = _const(256, 256, g, u, d)
    check(x, dy, "fp8 const %r" % ((g, u, d),))


def test_outliers_and_zero_rows_fp8():
    x, dy = make_inputs("t32768_h2048_outliers", device=DEV, T=3001)
    check(x, dy, "fp8 outliers T=3001")


def test_float8_dtype_outputs_and_int8_pass_unchanged():
    x, dy = random_inputs(256, 384, device=DEV, seed=5)
    T, H = dy.shape
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch has no float8_e4m3fn")
    outs = list(sq.empty_outputs(T, H, DEV, fp8=True))
    outs[0] = outs[0].view(torch.float8_e4m3fn)
    outs[2] = outs[2].view(torch.float8_e4m3fn)
    sq.silu_dot_fwd_bwd_quant_fuse_fp8(x, dy, *outs)
    torch.cuda.synchronize()
    got = [outs[0].view(torch.uint8).cpu().numpy(), outs[1].cpu().numpy(),
           outs[2].view(torch.uint8).cpu().numpy(), outs[3].cpu().numpy()]
    compare(got, oracle.silu_dot_fwd_bwd_quant_fuse_fp8(_bits(x), _bits(dy)), "fp8 dtype")
    # torch's own E4M3 decoding of the codes, times the scales, is within half
    # an E4M3 step (2^-4 relative, or 2^-10 * scale near zero) of the bf16
    # intermediates the oracle quantised
    dq = outs[0].float().cpu().numpy().reshape(T, -1, 128) * got[1][:, :, None]
    Y, D = oracle.intermediates(_bits(x), _bits(dy))
    ref = D.astype(np.float64).reshape(T, -1, 128)
    err = np.abs(dq - ref)
    assert np.all(err <= np.abs(ref) * 2.0**-4 + got[1][:, :, None] * 2.0**-10 * 1.0001)
    # the int8 pass, given int8 outputs, still rejects uint8 ones
    with pytest.raises(ValueError):
        sq.silu_dot_fwd_bwd_quant_fuse(x, dy, *sq.empty_outputs(T, H, DEV, fp8=True))
    with pytest.raises(ValueError):
        sq.silu_dot_fwd_bwd_quant_fuse_fp8(x, dy, *sq.empty_outputs(T, H, DEV))
