"""The forward quantisers at the token limits their header states (GPU).

silu_fwd_quant takes T up to 2^31 and the q8_1 forms (silu_fwd_quant_q8_1,
kquant_swiglu_q8_1_rows) rows up to 2^28.  At those sizes the oracle cannot
check every row, so the input is a block of P rows of seeded random values
repeated to the full size: the block's own outputs are first checked against
the oracle, and then every row of the full-size output must equal the
block's output for the same row of the block (a property of a row-wise
operation that holds at any size).  The outputs are poisoned first, so a row
that is never written fails.  The buffers take up to 88 GiB of device memory
and are freed after each case.
"""

import numpy as np
import pytest
import torch

import oracle
import swiglu_backward_int8_amd as sq
from swiglu_backward_int8_amd.inputs import random_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
P = 4096  # rows in the repeated block


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _all_rows_equal(big: torch.Tensor, block: torch.Tensor) -> bool:
    """Every P-row block of big equals block (compared on the device, in chunks)."""
    rows = big.shape[0]
    chunk = P * 16384
    for r0 in range(0, rows, chunk):
        part = big[r0:r0 + chunk]
        if not bool((part.view(-1, *block.shape) == block).all()):
            return False
    return True


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_forward_at_2_31_tokens():
    T, H = 2**31, 8  # x 64 GiB, codes 16 GiB, scales 8 GiB (one group per row)
    print("case forward T=2^31 H=8", flush=True)
    xs, _ = random_inputs(P, H, device=DEV, seed=31)
    yq_s = torch.empty((P, H), dtype=torch.int8, device=DEV)
    ys_s = torch.empty((P, 1), dtype=torch.float32, device=DEV)
    sq.silu_fwd_quant(xs, yq_s, ys_s)
    torch.cuda.synchronize()
    wq, ws = oracle.silu_fwd_quant(_bits(xs))
    assert np.array_equal(yq_s.cpu().numpy(), wq) and np.array_equal(ys_s.cpu().numpy(), ws)
    x = xs.repeat(T // P, 1)
    yq = torch.full((T, H), -7, dtype=torch.int8, device=DEV)
    ys = torch.full((T, 1), float("nan"), dtype=torch.float32, device=DEV)
    sq.silu_fwd_quant(x, yq, ys)
    torch.cuda.synchronize()
    del x
    assert _all_rows_equal(yq, yq_s), "codes"
    assert _all_rows_equal(ys, ys_s), "scales"


def test_q8_1_at_2_28_tokens():
    T, H = 2**28, 32  # x 32 GiB, blocks 9 GiB
    print("case q8_1 T=2^28 H=32", flush=True)
    xs, _ = random_inputs(P, H, device=DEV, seed=28)
    out_s = torch.empty((P, 36), dtype=torch.uint8, device=DEV)
    sq.silu_fwd_quant_q8_1(xs, out_s)
    torch.cuda.synchronize()
    assert np.array_equal(out_s.cpu().numpy(), oracle.silu_fwd_quant_q8_1(_bits(xs)))
    x = xs.repeat(T // P, 1)
    out = torch.full((T, 36), 0xA5, dtype=torch.uint8, device=DEV)
    sq.silu_fwd_quant_q8_1(x, out)
    torch.cuda.synchronize()
    del x
    assert _all_rows_equal(out, out_s)


def test_page_launch_shape_at_2_28_rows():
    rows, inter = 2**28, 32  # gate, up and h 16 GiB each, blocks 9 GiB
    print("case kquant_swiglu_q8_1_rows rows=2^28 inter=32", flush=True)
    xs, _ = random_inputs(P, inter, device=DEV, seed=29)
    gs, us = xs[:, :inter].contiguous(), xs[:, inter:].contiguous()
    w_s = torch.rand(P, device=DEV, generator=torch.Generator(device=DEV).manual_seed(3)) * 4 - 2
    out_s = torch.empty((P, 36), dtype=torch.uint8, device=DEV)
    h_s = torch.empty((P, inter), dtype=torch.bfloat16, device=DEV)
    sq.kquant_swiglu_q8_1_rows(gs, us, out_s, w=w_s, h_bf16=h_s)
    torch.cuda.synchronize()
    want, want_h = oracle.kquant_swiglu_q8_1_rows(_bits(gs), _bits(us), w_s.cpu().numpy())
    assert np.array_equal(out_s.cpu().numpy(), want) and np.array_equal(_bits(h_s), want_h)
    reps = rows // P
    gate, up, w = gs.repeat(reps, 1), us.repeat(reps, 1), w_s.repeat(reps)
    out = torch.full((rows, 36), 0xA5, dtype=torch.uint8, device=DEV)
    h = torch.full((rows, inter), float("nan"), dtype=torch.bfloat16, device=DEV)
    sq.kquant_swiglu_q8_1_rows(gate, up, out, w=w, h_bf16=h)
    torch.cuda.synchronize()
    del gate, up, w
    assert _all_rows_equal(out, out_s)
    assert _all_rows_equal(h.view(torch.int16), h_s.view(torch.int16))
