"""Parity of the forward quantiser's q8_1 block layout (silu_fwd_quant_q8_1)
with the CPU oracle (GPU): every block byte equal (codes, binary16 d and sum).
It is also checked against the library's own group-32 forward quantiser, and
the page's own launch shape (kquant_swiglu_q8_1_rows: separate gate and up,
the bf16 h written too) against the oracle.
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
    # every workload at its full token count
    print("case q8_1", name, flush=True)
    x, _ = make_inputs(name, device=DEV)
    check(x, label=name)


def test_block_sums_rounded_through_fp32():
    # A block's sum is fl32(scale * code sum) rounded to binary16.  Rounding
    # the exact product to binary16 once (what v_fma_mixlo_f16 does when the
    # compiler fuses the multiply into the conversion) gives another value for
    # some (scale, code sum) pairs, all with large code sums, which zero-mean
    # rows rarely reach.  Here every row is positive: a gate of 20 makes
    # silu(g) = g exactly, up is uniform in [0.1, 1) times a power of two per
    # row.  The oracle's codes and scales show how many blocks tell the two
    # roundings apart; the GPU must match the oracle's byte for byte.
    g = torch.Generator().manual_seed(11)
    T, H = 256, 4096
    up = (torch.rand(T, H, generator=g) * 0.9 + 0.1) * (2.0 ** torch.randint(-12, 4, (T, 1), generator=g).float())
    x = torch.cat([torch.full((T, H), 20.0), up], 1).bfloat16()
    q, s = oracle.silu_fwd_quant(_bits(x), group_size=32)[:2]
    qs = q.reshape(T, -1, 32).astype(np.int64).sum(-1)
    s = s.astype(np.float32)
    twice = (s * qs.astype(np.float32)).astype(np.float32).astype(np.float16).view(np.uint16)
    once = (s.astype(np.float64) * qs).astype(np.float16).view(np.uint16)
    differ = int((twice != once).sum())
    print("blocks whose sum depends on the rounding:", differ, flush=True)
    assert differ >= 20
    check(x.to(DEV), label="positive rows, T=%d H=%d" % (T, H))


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


def run_rows(gate, up, w=None, want_h=True):
    rows, inter = gate.shape
    out = torch.full((rows, (inter // 32) * sq.Q8_1_BLOCK), 0xA5, dtype=torch.uint8, device=DEV)
    h = torch.full((rows, inter), float("nan"), dtype=torch.bfloat16, device=DEV) if want_h else None
    sq.kquant_swiglu_q8_1_rows(gate, up, out, w=w, h_bf16=h)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (_bits(h) if want_h else None)


def check_rows(gate, up, w=None, want_h=True, label=""):
    got, h = run_rows(gate, up, w, want_h)
    want, want_h_bits = oracle.kquant_swiglu_q8_1_rows(_bits(gate), _bits(up), None if w is None else w.cpu().numpy())
    bad = int((got != want).sum())
    assert bad == 0, "%s: %d of %d block bytes differ" % (label, bad, got.size)
    if want_h:
        assert np.array_equal(h, want_h_bits), "%s: h differs" % label
    print("%s exact" % label, flush=True)


@pytest.mark.parametrize("name", ["t4096_h1408", "t32768_h2048_outliers"])
def test_page_launch_shape_workloads(name):
    # gate and up as separate arrays (copies of the workload's halves)
    x, _ = make_inputs(name, device=DEV)
    H = x.shape[1] // 2
    gate, up = x[:, :H].contiguous(), x[:, H:].contiguous()
    check_rows(gate, up, label=name + " separate gate/up")
    # byte-identical to the concatenated form, as the page says of the fused launch
    assert np.array_equal(run_rows(gate, up, want_h=False)[0], run(x))


@pytest.mark.parametrize("rows,inter", [(1, 32), (5, 96), (1000, 160), (129, 4096), (77, 2080)])
def test_page_launch_shape_with_and_without_weights(rows, inter):
    x, _ = random_inputs(rows, inter, device=DEV, seed=3 * rows + inter)
    gate, up = x[:, :inter].contiguous(), x[:, inter:].contiguous()
    w = torch.rand(rows, device=DEV, generator=torch.Generator(device=DEV).manual_seed(rows)) * 4 - 2
    check_rows(gate, up, label="rows=%d inter=%d" % (rows, inter))
    check_rows(gate, up, w=w, label="rows=%d inter=%d weighted" % (rows, inter))
    check_rows(gate, up, w=w, want_h=False, label="rows=%d inter=%d weighted, no h" % (rows, inter))


def test_page_launch_shape_same_array_for_gate_and_up():
    # the inputs are read only and may be one array: h = silu(g) * g
    x, _ = random_inputs(64, 256, device=DEV, seed=23)
    g = x[:, :256].contiguous()
    check_rows(g, g, label="gate == up")


def test_page_launch_shape_edges():
    rows, inter = 16, 128
    gate = torch.full((rows, inter), 20.0, dtype=torch.bfloat16, device=DEV)
    up = torch.ones((rows, inter), dtype=torch.bfloat16, device=DEV)
    gate[3] = 0.0
    up[5, :32] = torch.tensor([2.0**-130] * 31 + [0.0]).to(torch.bfloat16)
    up[7, 64:96] = 3.0e9
    check_rows(gate, up, label="edges")
    with pytest.raises(ValueError):
        sq.kquant_swiglu_q8_1_rows(gate[:, :48].contiguous(), up[:, :48].contiguous(),
                                   torch.empty((rows, 54), dtype=torch.uint8, device=DEV))
