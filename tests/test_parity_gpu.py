"""Parity of the HIP path with the CPU oracle (GPU).

Every case generates seeded inputs, runs the library through its C ABI (via the
thin binding), runs the oracle on the same bits, and compares element by
element.  The bar: every scale within 1e-6 relative of the oracle's, every int8
code equal except that |dq| == 1 is tolerated on at most 1e-4 of the codes of
each output (never more than 1).  The cases report how many codes differ; the
expected count is zero, because the kernel reproduces the oracle's arithmetic
operation for operation.
"""

import os

import numpy as np
import pytest
import torch

import oracle
import swiglu_backward_int8_amd as sq
from exact import all_finite_bf16
from swiglu_backward_int8_amd.inputs import WORKLOADS, make_inputs, random_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALE_RTOL = 1e-6
Q_FRACTION = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sq.lib()
    sq.prepare()


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_gpu(x, grad_y):
    T, H = grad_y.shape
    outs = sq.empty_outputs(T, H, x.device)
    for o in outs:  # poison: every element must be written
        o.fill_(-7 if o.dtype == torch.int8 else float("nan"))
    sq.silu_dot_fwd_bwd_quant_fuse(x, grad_y, *outs)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


def compare(got, want, label=""):
    names = ("grad_input_q", "grad_input_s", "y_q_t", "y_s_t")
    report = {}
    for name, g, w in zip(names, got, want):
        assert g.shape == w.shape, (name, g.shape, w.shape)
        if g.dtype == np.float32:
            assert not np.isnan(g).any(), "%s %s: unwritten scales" % (label, name)
            rel = np.abs(g.astype(np.float64) - w.astype(np.float64)) / np.maximum(np.abs(w.astype(np.float64)),
                                                                                1e-300)
            bad = int((rel > SCALE_RTOL).sum())
            report[name] = bad
            assert bad == 0, "%s %s: %d scales off, worst rel %g" % (label, name, bad, rel.max())
        else:
            d = np.abs(g.astype(np.int16) - w.astype(np.int16))
            n1 = int((d == 1).sum())
            report[name] = n1
            assert int(d.max(initial=0)) <= 1, "%s %s: |dq| up to %d" % (label, name, int(d.max()))
            assert n1 <= Q_FRACTION * d.size, "%s %s: %d codes off by one" % (label, name, n1)
    print("%s mismatches %s" % (label, report), flush=True)
    return report


def check(x, grad_y, label):
    got = run_gpu(x, grad_y)
    want = oracle.silu_dot_fwd_bwd_quant_fuse(_bits(x), _bits(grad_y))
    return compare(got, want, label)


def test_sigmoid_every_bf16_gate_bit_exact():
    bits = all_finite_bf16()
    gate = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    got = sq.eval_sigmoid(gate).cpu().numpy()
    want = np.array([oracle.sigmoid(oracle.bf16_to_f32(int(b))) for b in bits], dtype=np.float32)
    diff = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
    assert diff.size == 0, [(hex(int(bits[i])), float(got[i]), float(want[i])) for i in diff[:8]]


@pytest.mark.parametrize("name", ["t256_h256", "t4096_h1408", "t32768_h2048_outliers"])
def test_intermediates_bit_exact(name):
    T = 1024 if WORKLOADS[name].T > 4096 else None
    x, dy = make_inputs(name, device=DEV, T=T)
    y, d = sq.eval_intermediates(x, dy)
    Y, D = oracle.intermediates(_bits(x), _bits(dy))
    gy = (_bits(y).astype(np.uint32) << 16).view(np.float32)
    gd = (_bits(d).astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(gy.view(np.uint32), Y.view(np.uint32)), int((gy != Y).sum())
    assert np.array_equal(gd.view(np.uint32), D.view(np.uint32)), int((gd != D).sum())


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_parity(name):
    print("case", name, flush=True)
    x, dy = make_inputs(name, device=DEV)
    rep = check(x, dy, name)
    assert sum(rep.values()) == 0  # the kernel is expected to be exact


@pytest.mark.parametrize("name,seed", [("t256_h256", 1000), ("t4096_h1408", 1001), ("t8192_h4096", 1002),
                                       ("t16384_h11008", 1003), ("t32768_h2048_outliers", 1004)])
def test_workload_parity_second_seed(name, seed):
    print("case", name, seed, flush=True)
    x, dy = make_inputs(name, device=DEV, seed=seed)
    check(x, dy, "%s seed %d" % (name, seed))


@pytest.mark.parametrize("T,H,fp8", [(256, 256, False), (1000, 1376, False), (300, 1001, False), (256, 256, True)])
def test_bound_call_writes_what_the_plain_call_writes(T, H, fp8):
    # bind_backward checks the tensors once; each call of the bound function
    # must enqueue the same pass on the same buffers (called twice: the
    # second call rewrites every byte identically)
    x, dy = random_inputs(T, H, device=DEV, seed=T * 3 + H)
    plain = sq.empty_outputs(T, H, DEV, fp8=fp8)
    (sq.silu_dot_fwd_bwd_quant_fuse_fp8 if fp8 else sq.silu_dot_fwd_bwd_quant_fuse)(x, dy, *plain)
    bound_outs = sq.empty_outputs(T, H, DEV, fp8=fp8)
    run = sq.bind_backward(x, dy, *bound_outs, fp8=fp8)
    run()
    run()
    torch.cuda.synchronize()
    for a, b in zip(plain, bound_outs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("T,H", [(128, 128), (128, 1280), (1280, 128), (384, 640), (2048, 256)])
def test_shapes(T, H):
    x, dy = random_inputs(T, H, device=DEV, seed=T + H)
    check(x, dy, "T=%d H=%d" % (T, H))


def _const(T, H, g, u, d):
    x = torch.empty((T, 2 * H), dtype=torch.bfloat16, device=DEV)
    x[:, :H] = g
    x[:, H:] = u
    return x, torch.full((T, H), d, dtype=torch.bfloat16, device=DEV)


@pytest.mark.parametrize("g,u,d", [(0.0, 1.0, 1.0), (1.0, 1.0, 1.0), (20.0, 1.5, 0.25), (-2.0, 1.0, 1.0),
                                   (-100.0, 1.0, 1.0), (0.0, 0.0, 0.0)])
def test_constant_inputs(g, u, d):
    x, dy = _const(256, 256, g, u, d)
    check(x, dy, "const %r" % ((g, u, d),))


def test_saturated_gate_ties_to_even():
    T = H = 128
    x, dy = _const(T, H, 100.0, 0.0, 1.0)
    row = torch.tensor([127.0, 2.5, 0.5, -2.5, 126.5, 3.5, -0.5, 1.5], dtype=torch.bfloat16, device=DEV)
    x[:, H:H + 8] = row
    got = run_gpu(x, dy)
    assert got[0][0, :8].tolist() == [127, 2, 0, -2, 126, 4, 0, 2]
    check(x, dy, "ties")


@pytest.mark.parametrize("lo,hi", [(16.0, 17.5), (-90.0, -87.0), (-88.75, -87.5), (-1e-6, 1e-6)])
def test_gate_edge_ranges(lo, hi):
    # saturation edges, the subnormal-sigmoid band and the s == 1/2 band
    T, H = 256, 256
    gen = torch.Generator(device=DEV).manual_seed(99)
    g = lo + (hi - lo) * torch.rand((T, H), generator=gen, device=DEV)
    u = torch.randn((T, H), generator=gen, device=DEV)
    d = torch.randn((T, H), generator=gen, device=DEV)
    x = torch.cat([g, u], dim=1).to(torch.bfloat16).contiguous()
    check(x, d.to(torch.bfloat16), "gates in [%g, %g]" % (lo, hi))


def test_tiny_groups_overflowing_inverse():
    # Groups whose maximum is below 127 * 2^-128: 1/scale overflows to inf and
    # the clamp / zero rule decides the codes.  gate = 20 (s = 1), grad_y = 1,
    # so d_gate = up exactly.
    T = H = 128
    x, dy = _const(T, H, 20.0, 0.0, 1.0)
    tiny = torch.tensor([2.0**-130, -(2.0**-131), 0.0, 2.0**-133], dtype=torch.float32)
    x[:, H:H + 4] = tiny.to(torch.bfloat16).to(DEV)
    got = run_gpu(x, dy)
    assert got[0][0, :4].tolist() == [127, -127, 0, 127]  # every non-zero clamps
    check(x, dy, "tiny groups")


def test_zero_rows_and_outliers_small():
    x, dy = make_inputs("t32768_h2048_outliers", device=DEV, T=1024)
    rep = check(x, dy, "outliers T=1024")
    assert sum(rep.values()) == 0


def test_deterministic():
    x, dy = make_inputs("t4096_h1408", device=DEV)
    a = run_gpu(x, dy)
    b = run_gpu(x, dy)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_non_default_stream():
    x, dy = make_inputs("t4096_h1408", device=DEV)
    T, H = dy.shape
    s = torch.cuda.Stream(device=DEV)
    outs = sq.empty_outputs(T, H, DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        sq.silu_dot_fwd_bwd_quant_fuse(x, dy, *outs)
    s.synchronize()
    got = [o.cpu().numpy() for o in outs]
    compare(got, oracle.silu_dot_fwd_bwd_quant_fuse(_bits(x), _bits(dy)), "side stream")


@pytest.mark.parametrize("T,H", [(1, 128), (100, 256), (129, 128), (200, 384), (1000, 256), (1023, 128),
                                 (4097, 384), (16380, 256), (333, 1408)])
def test_ragged_token_counts(T, H):
    # the last token group holds T % 128 tokens; y_q_t rows are T bytes, so
    # T % 16 and T % 4 select the store width
    x, dy = random_inputs(T, H, device=DEV, seed=T * 7 + H)
    rep = check(x, dy, "ragged T=%d H=%d" % (T, H))
    assert sum(rep.values()) == 0


@pytest.mark.parametrize("T,H", [(32768, 4224), (8192 + 128, 4224), (8192, 8192), (4096, 2048)])
def test_tile_walk_orders(T, H):
    # rows of 33 tiles (longer than an XCD's share of 256 workgroups) over
    # 256 tile rows: the XCDs take interleaved tile rows with their own column
    # phase; over 65 tile rows (not a multiple of 8) only the phase applies;
    # rows of 64 and 16 tiles that deal out evenly: runs of 4 tiles (at 256
    # workgroups; other device sizes take the walks above)
    print("case walk T=%d H=%d" % (T, H), flush=True)
    x, dy = random_inputs(T, H, device=DEV, seed=T + H)
    assert sum(check(x, dy, "walk T=%d H=%d" % (T, H)).values()) == 0


def test_ragged_tokens_outlier_workload():
    x, dy = make_inputs("t32768_h2048_outliers", device=DEV, T=3001)
    rep = check(x, dy, "outliers T=3001")
    assert sum(rep.values()) == 0


def test_binding_rejects_bad_tensors():
    x, dy = random_inputs(128, 128, device=DEV)
    outs = list(sq.empty_outputs(128, 128, DEV))
    with pytest.raises(ValueError):
        sq.silu_dot_fwd_bwd_quant_fuse(x.float(), dy, *outs)
    with pytest.raises(ValueError):
        sq.silu_dot_fwd_bwd_quant_fuse(x, dy, outs[0], outs[1].double(), outs[2], outs[3])
    with pytest.raises(ValueError):
        sq.silu_dot_fwd_bwd_quant_fuse(x[:, :128], dy[:, :64], *outs)
    with pytest.raises(ValueError):
        x2, dy2 = random_inputs(200, 128, device=DEV)
        sq.silu_dot_fwd_bwd_quant_fuse(x2, dy2, *sq.empty_outputs(128, 128, DEV))
    with pytest.raises(ValueError):  # outputs for another H
        x3, dy3 = random_inputs(128, 100, device=DEV)
        sq.silu_dot_fwd_bwd_quant_fuse(x3, dy3, *sq.empty_outputs(128, 104, DEV))
    with pytest.raises(ValueError):
        sq.silu_dot_fwd_bwd_quant_fuse(x, dy, *outs, group_size=64)


def test_empty_inputs_are_no_ops():
    for T, H in ((0, 128), (128, 0)):
        x = torch.empty((T, 2 * H), dtype=torch.bfloat16, device=DEV)
        dy = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
        sq.silu_dot_fwd_bwd_quant_fuse(x, dy, *sq.empty_outputs(T, H, DEV))
    torch.cuda.synchronize()


def check_group(x, grad_y, group, label, fp8=False):
    """Parity for a group size other than 128: every code and scale bit-equal."""
    T, H = grad_y.shape
    outs = sq.empty_outputs(T, H, x.device, group=group, fp8=fp8)
    for o in outs:  # poison: every element must be written
        o.fill_(0x7F if o.dtype == torch.uint8 else -7 if o.dtype == torch.int8 else float("nan"))
    fn = sq.silu_dot_fwd_bwd_quant_fuse_fp8 if fp8 else sq.silu_dot_fwd_bwd_quant_fuse
    fn(x, grad_y, *outs, group_size=group)
    torch.cuda.synchronize()
    got = [o.cpu().numpy() for o in outs]
    ofn = oracle.silu_dot_fwd_bwd_quant_fuse_fp8 if fp8 else oracle.silu_dot_fwd_bwd_quant_fuse
    want = ofn(_bits(x), _bits(grad_y), group_size=group)
    for name, g, w in zip(("grad_input_q", "grad_input_s", "y_q_t", "y_s_t"), got, want):
        assert g.shape == w.shape, (label, name, g.shape, w.shape)
        gb, wb = g.view(np.uint8 if g.dtype.itemsize == 1 else np.uint32), w.view(np.uint8 if w.dtype.itemsize == 1 else np.uint32)
        bad = int((gb != wb).sum())
        assert bad == 0, "%s %s: %d of %d differ" % (label, name, bad, g.size)
    print("%s: bit-exact" % label, flush=True)


# Group sizes 64 and 32 divide the 128 x 128 tile; H need only be a multiple of
# the group, so the last channel block may hold 32, 64 or 96 channels.
@pytest.mark.parametrize("T,H,group", [(256, 256, 64), (256, 256, 32), (300, 192, 64), (1000, 160, 32),
                                       (129, 96, 32), (4096, 1408, 64), (2048, 1376, 32), (77, 64, 64),
                                       (1, 32, 32), (4100, 448, 64)])
def test_smaller_groups_and_ragged_h(T, H, group):
    print("case groups", T, H, group, flush=True)
    x, dy = random_inputs(T, H, device=DEV, seed=T + 3 * H + group)
    check_group(x, dy, group, "T=%d H=%d group=%d" % (T, H, group))


@pytest.mark.parametrize("group", [32, 64])
def test_smaller_groups_workloads(group):
    for name in ("t8192_h4096", "t32768_h2048_outliers"):
        print("case groups", name, group, flush=True)
        x, dy = make_inputs(name, device=DEV)
        check_group(x, dy, group, "%s group=%d" % (name, group))


@pytest.mark.parametrize("group", [32, 64])
def test_smaller_groups_fp8_and_overflowed_inverse(group):
    x, dy = random_inputs(640, 320, device=DEV, seed=group)
    check_group(x, dy, group, "fp8 T=640 H=320 group=%d" % group, fp8=True)
    # a group whose maximum is below 127 * 2^-128 (gate 20: d_gate == up)
    T, H = 128, 192
    x, dy = _const(T, H, 20.0, 0.0, 1.0)
    x[:, H:H + 4] = torch.tensor([2.0**-130, -(2.0**-131), 0.0, 2.0**-133], dtype=torch.float32).to(torch.bfloat16).to(DEV)
    check_group(x, dy, group, "tiny groups group=%d" % group)
    check_group(x, dy, group, "tiny groups fp8 group=%d" % group, fp8=True)


def test_group_size_errors():
    x, dy = random_inputs(128, 100, device=DEV)
    with pytest.raises(ValueError):  # scales shaped for group 128
        sq.silu_dot_fwd_bwd_quant_fuse(x, dy, *sq.empty_outputs(128, 100, DEV), group_size=64)
    x, dy = random_inputs(128, 96, device=DEV)
    with pytest.raises(ValueError):
        sq.silu_dot_fwd_bwd_quant_fuse(x, dy, *sq.empty_outputs(128, 96, DEV, group=32), group_size=48)


# H not a multiple of the group (any multiple of 8): one row group holds the
# last H % group channels of d_gate and the first of d_up, the d_up groups sit
# shifted against the 128-channel blocks, and the row's last group may be
# partial.  Shapes cover r = H % group from 8 to 120, H below the group, and
# windows that need one block more than the channels (r > 128 - H % 128).
# With H > 128 the d_up halves are handed along runs of blocks (any group):
# r = 8 .. 120 with r / 8 odd and even (the window's lane pairs differ), runs
# of one block (small T) and of three or four (T = 8192, H = 1376 and
# T = 4096, H = 11000), and window n present (r > 64) or not.
@pytest.mark.parametrize("T,H,group", [(256, 200, 128), (129, 40, 32), (64, 8, 128), (300, 1000, 128),
                                       (1000, 1064, 64), (128, 136, 128), (4096, 1400, 128), (333, 520, 32),
                                       (77, 2056, 64), (1, 24, 32), (130, 248, 128), (640, 11000, 128),
                                       (256, 1376, 128), (200, 272, 128), (129, 704, 128), (300, 848, 128),
                                       (1000, 176, 128), (8192, 1376, 128), (4096, 11000, 128), (1500, 2752, 128),
                                       (8192, 1376, 64), (4096, 11000, 32), (3000, 2744, 64), (640, 1064, 32)])
def test_straddling_groups(T, H, group):
    print("case straddle", T, H, group, flush=True)
    x, dy = random_inputs(T, H, device=DEV, seed=5 * T + H + group)
    check_group(x, dy, group, "straddle T=%d H=%d group=%d" % (T, H, group))


@pytest.mark.parametrize("T,H,group", [(256, 200, 128), (300, 1000, 64), (129, 40, 32), (8192, 1376, 128)])
def test_straddling_groups_fp8(T, H, group):
    print("case straddle fp8", T, H, group, flush=True)
    x, dy = random_inputs(T, H, device=DEV, seed=T + H + group)
    check_group(x, dy, group, "straddle fp8 T=%d H=%d group=%d" % (T, H, group), fp8=True)


@pytest.mark.parametrize("group", [32, 128])
def test_straddling_groups_edge_values(group):
    # saturated gate, u = d = 1: d_gate = 1 and d_up = 20, so the straddling
    # group's maximum comes from the d_up side; then a straddling group of
    # tiny values whose inverse overflows, and zero rows
    T, H = 256, 40 if group == 32 else 200
    x, dy = _const(T, H, 20.0, 1.0, 1.0)
    check_group(x, dy, group, "straddle const group=%d" % group)
    check_group(x, dy, group, "straddle const fp8 group=%d" % group, fp8=True)
    r = H % group
    x, dy = _const(T, H, 20.0, 0.0, 1.0)  # d_gate = d u = 0, d_up = 20 d
    tiny = torch.tensor([2.0**-130, -(2.0**-131), 0.0, 2.0**-133], dtype=torch.float32).to(torch.bfloat16).to(DEV)
    x[:, 2 * H - 4:] = tiny  # up at d_gate's last channels: d_gate (and y) tiny there
    dy[:, :group - r] = 0.0  # d_up's share of the straddling group is zero
    x[7] = 0.0
    dy[9] = 0.0
    check_group(x, dy, group, "straddle tiny group=%d" % group)
    check_group(x, dy, group, "straddle tiny fp8 group=%d" % group, fp8=True)


# Shapes drawn at random (a fixed seed, so the list is the same every run):
# T and H anywhere up to 2500, every group size, both code formats; H picks
# up every residue class the kernels branch on (multiple of the group, of 8
# only, odd), and T ragged or not.
def _random_shapes(n=18, seed=20260):
    rng = np.random.default_rng(seed)
    shapes = []
    for i in range(n):
        group = int(rng.choice([32, 64, 128]))
        kind = i % 3
        H = int(rng.integers(1, 2500))
        if kind == 0:
            H = max(group, H - H % group)  # a multiple of the group
        elif kind == 1:
            H = max(8, H - H % 8)          # a multiple of 8
        T = int(rng.integers(1, 2500))
        shapes.append((T, H, group, bool(i % 2)))
    return shapes


@pytest.mark.parametrize("T,H,group,fp8", _random_shapes())
def test_random_shapes(T, H, group, fp8):
    print("case random", T, H, group, fp8, flush=True)
    x, dy = random_inputs(T, H, device=DEV, seed=T * 7919 + H)
    check_group(x, dy, group, "random T=%d H=%d group=%d fp8=%d" % (T, H, group, fp8), fp8=fp8)


def test_hip_graph_capture_and_replay():
    # Each entry point is one kernel launch on the caller's stream, so once the
    # sigmoid table exists the calls can be captured in a HIP graph.  The graph
    # (pass, forward quantiser, GEMM on the pass's codes) is replayed on new
    # inputs copied into the captured buffers, with eager work in between;
    # every replay must match the oracle.
    T, H, D = 512, 1408, 256
    sq.prepare()
    x, dy = random_inputs(T, H, device=DEV, seed=41)
    outs = sq.empty_outputs(T, H, DEV)
    yq = torch.empty((T, H), dtype=torch.int8, device=DEV)
    ys = torch.empty((T, H // 128), dtype=torch.float32, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(5)
    W = torch.randint(-127, 128, (D, 2 * H), dtype=torch.int8, device=DEV, generator=gen)
    sW = torch.rand((D // 128, 2 * H // 128), device=DEV, generator=gen)
    C = torch.empty((T, D), dtype=torch.float32, device=DEV)

    def calls():
        sq.silu_dot_fwd_bwd_quant_fuse(x, dy, *outs)
        sq.silu_fwd_quant(x, yq, ys)
        sq.i8_gemm_group_scaled(outs[0], outs[1], W, sW, C, b_rows_per_scale=128)

    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # a warm-up outside the capture
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for seed in (42, 43, 44):
        x2, dy2 = random_inputs(T, H, device=DEV, seed=seed)
        x.copy_(x2)
        dy.copy_(dy2)
        for o in outs + (yq, ys, C):
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        compare([o.cpu().numpy() for o in outs], oracle.silu_dot_fwd_bwd_quant_fuse(_bits(x2), _bits(dy2)),
                "graph replay %d" % seed)
        wq, ws = oracle.silu_fwd_quant(_bits(x2))
        assert np.array_equal(yq.cpu().numpy(), wq) and np.array_equal(ys.cpu().numpy(), ws)
        want, want_abs = oracle.i8_gemm_group_scaled(outs[0].cpu().numpy(), outs[1].cpu().numpy(), W.cpu().numpy(),
                                                     sW.cpu().numpy(), b_rows_per_scale=128)
        assert np.all(np.abs(C.cpu().numpy() - want) <= (2 * H // 128 + 2) * 2.0**-24 * want_abs)


@pytest.mark.parametrize("H", [1376, 1001])
def test_hip_graph_replay_of_the_other_kernels(H):
    # The kernels for H not a multiple of the group (1376: runs of blocks) and
    # of 8 (1001: the two-team position tiles; the forward quantiser's shifted
    # pieces) captured with the pass's entry points and replayed on new inputs.
    T = 640
    x, dy = random_inputs(T, H, device=DEV, seed=47)
    outs = sq.empty_outputs(T, H, DEV)
    yq = torch.empty((T, H), dtype=torch.int8, device=DEV)
    ys = torch.empty((T, -(-H // 128)), dtype=torch.float32, device=DEV)
    yb = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)

    def calls():
        sq.silu_dot_fwd_bwd_quant_fuse(x, dy, *outs)
        sq.silu_fwd_quant(x, yq, ys, y_bf16=yb)

    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for seed in (48, 49, 50):
        x2, dy2 = random_inputs(T, H, device=DEV, seed=seed)
        x.copy_(x2)
        dy.copy_(dy2)
        for o in outs + (yq, ys, yb):
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        compare([o.cpu().numpy() for o in outs], oracle.silu_dot_fwd_bwd_quant_fuse(_bits(x2), _bits(dy2)),
                "graph replay H=%d %d" % (H, seed))
        wq, ws, wb = oracle.silu_fwd_quant(_bits(x2), want_bf16=True)
        assert np.array_equal(yq.cpu().numpy(), wq) and np.array_equal(ys.cpu().numpy(), ws)
        assert np.array_equal(_bits(yb), wb)


# H not a multiple of 8: rows start off 16 bytes (loads take aligned pieces and
# shift them, code stores write aligned pieces and the tile's own bytes at both
# ends); groups still straddle d_gate and d_up.
@pytest.mark.parametrize("T,H,group", [(256, 100, 128), (129, 1, 32), (64, 3, 128), (300, 1001, 64),
                                       (1000, 2050, 128), (77, 13, 32), (4096, 1410, 128), (1, 250, 64)])
def test_h_not_a_multiple_of_8(T, H, group):
    print("case narrow", T, H, group, flush=True)
    x, dy = random_inputs(T, H, device=DEV, seed=7 * T + H + group)
    check_group(x, dy, group, "narrow T=%d H=%d group=%d" % (T, H, group))


# The tiled path over position tiles of [d_gate | d_up]: the tile that holds
# position H with r = H mod 128 of 1, 63, 65 and 127 (a last tile of less or
# more than half a tile), a row of 86 channel tiles, and seeded random shapes.
@pytest.mark.parametrize("T,H,group", [(300, 129, 128), (260, 255, 64), (130, 191, 32), (129, 193, 128),
                                       (2048, 11001, 128), (512, 11003, 32)])
def test_h_not_a_multiple_of_8_position_tiles(T, H, group):
    print("case narrow tiles", T, H, group, flush=True)
    x, dy = random_inputs(T, H, device=DEV, seed=3 * T + H + group)
    check_group(x, dy, group, "narrow tiles T=%d H=%d group=%d" % (T, H, group))


def _random_narrow_shapes(n=12, seed=8081):
    rng = np.random.default_rng(seed)
    shapes = []
    for i in range(n):
        group = int(rng.choice([32, 64, 128]))
        H = int(rng.integers(1, 3000))
        if H % 8 == 0:
            H += int(rng.integers(1, 8))
        T = int(rng.integers(1, 1500))
        shapes.append((T, H, group, bool(i % 2)))
    return shapes


@pytest.mark.parametrize("T,H,group,fp8", _random_narrow_shapes())
def test_h_not_a_multiple_of_8_random(T, H, group, fp8):
    print("case narrow random", T, H, group, fp8, flush=True)
    x, dy = random_inputs(T, H, device=DEV, seed=T * 31 + H)
    check_group(x, dy, group, "narrow random T=%d H=%d group=%d fp8=%d" % (T, H, group, fp8), fp8=fp8)


@pytest.mark.parametrize("T,H,group", [(256, 100, 128), (300, 1001, 32)])
def test_h_not_a_multiple_of_8_fp8_and_edges(T, H, group):
    x, dy = random_inputs(T, H, device=DEV, seed=T + H)
    check_group(x, dy, group, "narrow fp8 T=%d H=%d group=%d" % (T, H, group), fp8=True)
    # a saturated gate, a group of tiny values whose inverse overflows, zero rows
    x, dy = _const(T, H, 20.0, 0.0, 1.0)
    tiny = torch.tensor([2.0**-130, -(2.0**-131), 0.0, 2.0**-133], dtype=torch.float32).to(torch.bfloat16).to(DEV)
    x[:, 2 * H - 4:] = tiny
    dy[:, :group] = 0.0
    x[7] = 0.0
    dy[9] = 0.0
    check_group(x, dy, group, "narrow tiny T=%d H=%d group=%d" % (T, H, group))
    check_group(x, dy, group, "narrow tiny fp8 T=%d H=%d group=%d" % (T, H, group), fp8=True)
