"""The largest shapes the entry points accept (GPU).

The byte offsets inside a tile, the buffer record counts and the tile indices
are 32-bit: these cases run each entry point at (or next to) the limit its
header states and compare slices of the outputs with the oracle run on the
same slices of the inputs.  Token rows, 128-token groups and 128-channel
groups are independent of each other, so a slice of 256 tokens (or channels)
aligned to 128 has exactly the oracle's outputs for those tokens (channels).
"""

import numpy as np
import pytest
import torch

import oracle
import swiglu_backward_int8_amd as sq

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available()
    sq.prepare()


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _inputs(T, H, seed):
    gen = torch.Generator(device=DEV).manual_seed(seed)
    x = torch.randn((T, 2 * H), generator=gen, device=DEV).to(torch.bfloat16)
    dy = (torch.randn((T, H), generator=gen, device=DEV) * 0.01).to(torch.bfloat16)
    return x, dy


def _equal(label, got, want):
    for name, g, w in zip(("grad_input_q", "grad_input_s", "y_q_t", "y_s_t"), got, want):
        gb = g.view(np.uint8 if g.dtype.itemsize == 1 else np.uint32)
        wb = w.view(np.uint8 if w.dtype.itemsize == 1 else np.uint32)
        assert g.shape == w.shape and np.array_equal(gb, wb), "%s %s: %d differ" % (label, name, int((gb != wb).sum()))


def test_backward_at_the_token_limit():
    # T = 2^23 (the largest T), H = 128: y_q_t rows are 8 MiB long
    T, H = 1 << 23, 128
    print("case T=2^23 H=128", flush=True)
    x, dy = _inputs(T, H, 1)
    gq, gs, yq, ys = sq.empty_outputs(T, H, DEV)
    sq.silu_dot_fwd_bwd_quant_fuse(x, dy, gq, gs, yq, ys)
    torch.cuda.synchronize()
    for t0 in (0, T // 2 + 128, T - 256):
        want = oracle.silu_dot_fwd_bwd_quant_fuse(_bits(x[t0:t0 + 256]), _bits(dy[t0:t0 + 256]))
        got = (gq[t0:t0 + 256].cpu().numpy(), gs[t0:t0 + 256].cpu().numpy(),
               yq[:, t0:t0 + 256].cpu().numpy(), ys[:, t0 // 128:t0 // 128 + 2].cpu().numpy())
        _equal("T=2^23 tokens %d.." % t0, got, want)
    del x, dy, gq, gs, yq, ys
    torch.cuda.empty_cache()


def test_backward_at_the_channel_limit():
    # H = 2^22 (the largest H), T = 128: a lane's offset in x reaches 2^31 - 16
    T, H = 128, 1 << 22
    print("case T=128 H=2^22", flush=True)
    x, dy = _inputs(T, H, 2)
    gq, gs, yq, ys = sq.empty_outputs(T, H, DEV)
    sq.silu_dot_fwd_bwd_quant_fuse(x, dy, gq, gs, yq, ys)
    torch.cuda.synchronize()
    for h0 in (0, H // 2 + 128, H - 256):
        xs = torch.cat([x[:, h0:h0 + 256], x[:, H + h0:H + h0 + 256]], dim=1)
        want = oracle.silu_dot_fwd_bwd_quant_fuse(_bits(xs), _bits(dy[:, h0:h0 + 256]))
        g0, g1 = h0 // 128, (H + h0) // 128
        got = (torch.cat([gq[:, h0:h0 + 256], gq[:, H + h0:H + h0 + 256]], dim=1).cpu().numpy(),
               torch.cat([gs[:, g0:g0 + 2], gs[:, g1:g1 + 2]], dim=1).cpu().numpy(),
               yq[h0:h0 + 256].cpu().numpy(), ys[h0:h0 + 256].cpu().numpy())
        _equal("H=2^22 channels %d.." % h0, got, want)
    del x, dy, gq, gs, yq, ys
    torch.cuda.empty_cache()


def test_backward_past_the_limits_is_rejected():
    # shapes past the limits are refused before any device work
    for T, H in (((1 << 23) + 1, 128), (128, (1 << 22) + 128)):
        assert sq.raw_call(1 << 40, 2 << 40, 3 << 40, 4 << 40, 5 << 40, 6 << 40, T, H, 128, 0) == 2


def test_forward_at_the_channel_limit():
    T, H = 128, 1 << 22
    print("case forward T=128 H=2^22", flush=True)
    x, _ = _inputs(T, H, 3)
    yq = torch.empty((T, H), dtype=torch.int8, device=DEV)
    ys = torch.empty((T, H // 128), dtype=torch.float32, device=DEV)
    sq.silu_fwd_quant(x, yq, ys)
    torch.cuda.synchronize()
    for h0 in (0, H - 256):
        xs = torch.cat([x[:, h0:h0 + 256], x[:, H + h0:H + h0 + 256]], dim=1)
        wq, ws = oracle.silu_fwd_quant(_bits(xs))
        assert np.array_equal(yq[:, h0:h0 + 256].cpu().numpy(), wq)
        assert np.array_equal(ys[:, h0 // 128:h0 // 128 + 2].cpu().numpy().view(np.uint32), ws.view(np.uint32))
    del x, yq, ys
    torch.cuda.empty_cache()


def test_forward_h_not_a_multiple_of_8_at_the_limits():
    # the shifted tiled path at H = 2^22 - 1 (T = 64: the last unit of a row is
    # 127 channels) and at T = 2^25 with H = 3 (every unit one partial
    # group; the aligned bases of y_q and y_bf16 lie below rows far past 2^32
    # bytes of x)
    for T, H, G, rows, cols in ((64, (1 << 22) - 1, 128, None, (0, (1 << 22) - 1 - 300)),
                                (1 << 25, 3, 32, (0, (1 << 24) + 5, (1 << 25) - 300), None)):
        print("case forward narrow T=%d H=%d" % (T, H), flush=True)
        x, _ = _inputs(T, H, 9)
        yq = torch.empty((T, H), dtype=torch.int8, device=DEV)
        ys = torch.empty((T, -(-H // G)), dtype=torch.float32, device=DEV)
        yb = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
        sq.silu_fwd_quant(x, yq, ys, y_bf16=yb, group_size=G)
        torch.cuda.synchronize()
        if cols is not None:
            for h0 in cols:  # whole groups: h0 multiple of G, or the row's last 300 channels from a group start
                h0 = h0 - h0 % G
                n = min(H - h0, 384)
                xs = torch.cat([x[:, h0:h0 + n], x[:, H + h0:H + h0 + n]], dim=1)
                wq, ws, wb = oracle.silu_fwd_quant(_bits(xs), group_size=G, want_bf16=True)
                assert np.array_equal(yq[:, h0:h0 + n].cpu().numpy(), wq), h0
                g0 = h0 // G
                assert np.array_equal(ys[:, g0:g0 + ws.shape[1]].cpu().numpy().view(np.uint32), ws.view(np.uint32)), h0
                assert np.array_equal(_bits(yb[:, h0:h0 + n]), wb), h0
        else:
            for t0 in rows:
                xs = x[t0:t0 + 300]
                wq, ws, wb = oracle.silu_fwd_quant(_bits(xs), group_size=G, want_bf16=True)
                assert np.array_equal(yq[t0:t0 + 300].cpu().numpy(), wq), t0
                assert np.array_equal(ys[t0:t0 + 300].cpu().numpy().view(np.uint32), ws.view(np.uint32)), t0
                assert np.array_equal(_bits(yb[t0:t0 + 300]), wb), t0
        del x, yq, ys, yb
        torch.cuda.empty_cache()


def test_gemm_at_the_k_limit():
    # K = 2^22 (the largest K): a tile's rows of A span 2^29 bytes of one buffer
    M, N, K = 256, 256, 1 << 22
    print("case GEMM K=2^22", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(4)
    A = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=DEV, generator=gen)
    B = torch.randint(-127, 128, (N, K), dtype=torch.int8, device=DEV, generator=gen)
    sA = torch.rand((M, K // 128), device=DEV, generator=gen) * 1e-4
    sB = torch.rand((N, K // 128), device=DEV, generator=gen) * 1e-4
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    sq.i8_gemm_group_scaled(A, sA, B, sB, C)
    torch.cuda.synchronize()
    rows, cols = [0, 129, 255], [1, 200, 255]
    want, want_abs = oracle.i8_gemm_group_scaled(A[rows].cpu().numpy(), sA[rows].cpu().numpy(),
                                                 B[cols].cpu().numpy(), sB[cols].cpu().numpy())
    got = C[rows][:, cols].cpu().numpy().astype(np.float64)
    bound = (K // 128 + 2) * 2.0**-24 * want_abs
    assert np.all(np.abs(got - want) <= bound), (got, want)


def test_straddling_kernel_at_the_channel_limit():
    # H = 2^22 - 8 with group 128: r = 120, so 32,768 blocks per token block
    # are walked in runs of four, a last window (the final r channels of d_up,
    # r > 64) follows the last block, and a lane's offset in x comes close to
    # 2^31.  The first 256 and the last 256 channels of the row are checked:
    # the straddling group holds d_gate's last 120 channels and d_up's first 8.
    T, H, G = 128, (1 << 22) - 8, 128
    print("case straddle T=128 H=2^22-8", flush=True)
    x, dy = _inputs(T, H, 5)
    gq, gs, yq, ys = sq.empty_outputs(T, H, DEV, group=G)
    sq.silu_dot_fwd_bwd_quant_fuse(x, dy, gq, gs, yq, ys, group_size=G)
    torch.cuda.synchronize()
    _, D = oracle.intermediates(_bits(torch.cat([x[:, H - 256:H], x[:, 2 * H - 256:]], dim=1)),
                                _bits(dy[:, H - 256:]))
    _, D0 = oracle.intermediates(_bits(torch.cat([x[:, :256], x[:, H:H + 256]], dim=1)), _bits(dy[:, :256]))
    # concatenated row positions H - 120 .. H + 7: d_gate's last 120, d_up's first 8
    j = (H - 120) // G
    gq_np, gs_np = gq.cpu().numpy(), gs.cpu().numpy()
    for t in range(T):
        seg = np.concatenate([D[t, 256 - 120:256], D0[t, 256:256 + 8]])
        q, s = oracle.quant_group(seg)
        assert s == gs_np[t, j] and np.array_equal(q, gq_np[t, H - 120:H + 8]), t
        # the last group of the row: d_up's last 2H - (H + 8) = H - 8 ... its
        # final (2H) % 128 = 112 positions
        n = (2 * H) % G
        q, s = oracle.quant_group(D[t, 512 - n:512])
        assert s == gs_np[t, -1] and np.array_equal(q, gq_np[t, 2 * H - n:]), t
    del x, dy, gq, gs, yq, ys
    torch.cuda.empty_cache()


def test_straddling_kernel_at_the_token_limit():
    # T = 2^23, H = 8, group 32: every row is a single partial group of 16
    # (8 of d_gate, 8 of d_up), in one block; y_q_t rows are 8 MiB long
    T, H, G = 1 << 23, 8, 32
    print("case straddle T=2^23 H=8", flush=True)
    x, dy = _inputs(T, H, 6)
    gq, gs, yq, ys = sq.empty_outputs(T, H, DEV, group=G)
    sq.silu_dot_fwd_bwd_quant_fuse(x, dy, gq, gs, yq, ys, group_size=G)
    torch.cuda.synchronize()
    for t0 in (0, T // 2 + 96, T - 256):
        want = oracle.silu_dot_fwd_bwd_quant_fuse(_bits(x[t0:t0 + 256]), _bits(dy[t0:t0 + 256]), group_size=G)
        got = (gq[t0:t0 + 256].cpu().numpy(), gs[t0:t0 + 256].cpu().numpy(),
               yq[:, t0:t0 + 256].cpu().numpy(), ys[:, t0 // G:t0 // G + 256 // G].cpu().numpy())
        _equal("straddle T=2^23 tokens %d.." % t0, got, want)
    del x, dy, gq, gs, yq, ys
    torch.cuda.empty_cache()


def test_narrow_kernels_at_the_token_limit():
    # T = 2^23, H = 3 (not a multiple of 8: the position-tile kernel), group
    # 32: every row is one partial group of 6; y_q_t rows are 8 MiB long
    T, H, G = 1 << 23, 3, 32
    print("case narrow T=2^23 H=3", flush=True)
    x, dy = _inputs(T, H, 7)
    gq, gs, yq, ys = sq.empty_outputs(T, H, DEV, group=G)
    sq.silu_dot_fwd_bwd_quant_fuse(x, dy, gq, gs, yq, ys, group_size=G)
    torch.cuda.synchronize()
    for t0 in (0, T // 2 + 64, T - 256):
        want = oracle.silu_dot_fwd_bwd_quant_fuse(_bits(x[t0:t0 + 256]), _bits(dy[t0:t0 + 256]), group_size=G)
        got = (gq[t0:t0 + 256].cpu().numpy(), gs[t0:t0 + 256].cpu().numpy(),
               yq[:, t0:t0 + 256].cpu().numpy(), ys[:, t0 // G:t0 // G + 256 // G].cpu().numpy())
        _equal("narrow T=2^23 tokens %d.." % t0, got, want)
    del x, dy, gq, gs, yq, ys
    torch.cuda.empty_cache()


def test_narrow_kernels_at_the_channel_limit():
    # H = 2^22 - 1 with group 128: r = 127, so the straddling group holds
    # d_gate's last 127 channels and d_up's first one, and the row's last
    # group is d_up's final 126 channels.  T = 64 is one partial token group.
    T, H, G = 64, (1 << 22) - 1, 128
    print("case narrow T=64 H=2^22-1", flush=True)
    x, dy = _inputs(T, H, 8)
    gq, gs, yq, ys = sq.empty_outputs(T, H, DEV, group=G)
    sq.silu_dot_fwd_bwd_quant_fuse(x, dy, gq, gs, yq, ys, group_size=G)
    torch.cuda.synchronize()
    Y1, D1 = oracle.intermediates(_bits(torch.cat([x[:, H - 256:H], x[:, 2 * H - 256:]], dim=1)),
                                  _bits(dy[:, H - 256:]))
    Y0, D0 = oracle.intermediates(_bits(torch.cat([x[:, :256], x[:, H:H + 256]], dim=1)), _bits(dy[:, :256]))
    r, n = H % G, (2 * H) % G
    j = (H - r) // G
    head_q, head_s = gq[:, :256].cpu().numpy(), gs[:, :2].cpu().numpy()
    mid_q, mid_s = gq[:, H - r:H - r + G].cpu().numpy(), gs[:, j].cpu().numpy()
    tail_q, tail_s = gq[:, 2 * H - n:].cpu().numpy(), gs[:, -1].cpu().numpy()
    for t in range(T):
        for k in range(2):
            q, s = oracle.quant_group(D0[t, 128 * k:128 * k + 128])
            assert s == head_s[t, k] and np.array_equal(q, head_q[t, 128 * k:128 * k + 128]), (t, k)
        q, s = oracle.quant_group(np.concatenate([D1[t, 256 - r:256], D0[t, 256:256 + G - r]]))
        assert s == mid_s[t] and np.array_equal(q, mid_q[t]), t
        q, s = oracle.quant_group(D1[t, 512 - n:512])
        assert s == tail_s[t] and np.array_equal(q, tail_q[t]), t
    for Y, c0 in ((Y0, 0), (Y1, H - 256)):
        yq_np, ys_np = yq[c0:c0 + 256].cpu().numpy(), ys[c0:c0 + 256, 0].cpu().numpy()
        for c in range(256):
            q, s = oracle.quant_group(Y[:, c])
            assert s == ys_np[c] and np.array_equal(q, yq_np[c]), c0 + c
    del x, dy, gq, gs, yq, ys
    torch.cuda.empty_cache()
