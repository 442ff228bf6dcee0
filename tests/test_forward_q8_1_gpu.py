"""Parity of the forward quantiser's q8_1 block layout (silu_fwd_quant_q8_1)
with the CPU oracle (GPU): every block byte equal (codes, binary16 d and sum).
It is also checked against the library's own group-32 forward quantiser.
"""

import numpy as np
import pytest
import torch

import oracle
import swiglu_backward_int8_amd as sq
from swiglu_backward_int8_amd.inputs import WORKLOADS, make_inputs, random_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available()
    sq.prepare()


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run(x, w=None):
    T, H = x.shape[0], x.shape[1] // 2
    out = torch.full((T, (H // 32) * sq.Q8_1_BLOCK), 0xA5, dtype=torch.uint8, device=DEV)  # all written
    sq.silu_fwd_quant_q8_1(x, out, row_weight=w)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(x, w=None, label=""):
    got = run(x, w)
    want = oracle.silu_fwd_quant_q8_1(_bits(x), None if w is None else w.cpu().numpy())
    bad = int((got != want).sum())
    assert bad == 0, "%s: %d of %d bytes differ" % (label, bad, got.size)
    print("%s exact" % label, flush=True)
    return got


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workloads(name):
    T = min(WORKLOADS[name].T, 4096)
    x, _ = make_inputs(name, device=DEV, T=T)
    check(x, label=name)


@pytest.mark.parametrize("T,H", [(1, 32), (5, 96), (1000, 160), (129, 4096), (77, 2080)])
def test_shapes_with_and_without_weights(T, H):
    x, _ = random_inputs(T, H, device=DEV, seed=T + H)
    w = torch.rand(T, device=DEV, generator=torch.Generator(device=DEV).manual_seed(T)) * 4 - 2
    check(x, label="T=%d H=%d" % (T, H))
    check(x, w=w, label="T=%d H=%d weighted" % (T, H))


def test_matches_the_group_32_forward_quantiser():
    T, H = 256, 1408
    x, _ = make_inputs("t4096_h1408", device=DEV, T=T)
    got = run(x)
    d, s, q = oracle.split_q8_1(got)
    yq = torch.empty((T, H), dtype=torch.int8, device=DEV)
    ys = torch.empty((T, H // 32), dtype=torch.float32, device=DEV)
    sq.silu_fwd_quant(x, yq, ys, group_size=32)
    torch.cuda.synchronize()
    assert np.array_equal(q.reshape(T, H), yq.cpu().numpy())
    assert np.array_equal(d, ys.cpu().numpy().astype(np.float16))


def test_edge_values():
    # saturated gate (all codes 127), zero rows (d = 1, sum = 0), a tiny group
    # whose inverse overflows (d underflows to 0 in binary16), outliers whose
    # scale overflows binary16 (d = inf)
    T, H = 64, 256
    x = torch.empty((T, 2 * H), dtype=torch.bfloat16, device=DEV)
    x[:, :H] = 20.0
    x[:, H:] = 1.0
    x[3] = 0.0
    x[5, H:H + 32] = torch.tensor([2.0**-130] * 31 + [0.0]).to(torch.bfloat16)
    x[5, :32] = 20.0
    x[7, H + 64:H + 96] = 3.0e9
    got = check(x, label="edges")
    d, s, q = oracle.split_q8_1(got)
    assert d[3, 0] == 1.0 and s[3, 0] == 0.0 and not q[3].any()
    assert np.isinf(d[7, 2])


def test_errors():
    x, _ = random_inputs(8, 48, device=DEV)
    with pytest.raises(ValueError):  # H not a multiple of 32
        sq.silu_fwd_quant_q8_1(x, torch.empty((8, 54), dtype=torch.uint8, device=DEV))
    x, _ = random_inputs(8, 64, device=DEV)
    with pytest.raises(ValueError):  # wrong block array shape
        sq.silu_fwd_quant_q8_1(x, torch.empty((8, 64), dtype=torch.uint8, device=DEV))
    sq.silu_fwd_quant_q8_1(torch.empty((0, 128), dtype=torch.bfloat16, device=DEV),
                           torch.empty((0, 72), dtype=torch.uint8, device=DEV))


def test_block_base_only_4_byte_aligned():
    # the blocks may start 4 bytes into an allocation: the 16-byte store path
    # is then not taken
    T, H = 40, 256
    x, _ = random_inputs(T, H, device=DEV, seed=17)
    raw = torch.full((T * (H // 32) * 36 + 16,), 0xA5, dtype=torch.uint8, device=DEV)
    out = raw[4:4 + T * (H // 32) * 36].view(T, -1)
    sq.silu_fwd_quant_q8_1(x, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.silu_fwd_quant_q8_1(_bits(x)))
    r = raw.cpu().numpy()
    assert np.all(r[:4] == 0xA5) and np.all(r[4 + T * (H // 32) * 36:] == 0xA5)
