"""Parity of the group-scaled int8 GEMM (matrix cores) with the CPU oracle (GPU).

The oracle gives the exact value C and the sum of the absolute group terms
C_abs.  The kernel adds the groups in ascending order in fp32, each as
fma(float(dot), fl(sA * sB), acc): one rounding of the scale product and one
of each fused step, so |C_gpu - C| <= (groups + 1) * 2^-24 * C_abs.  The test
allows (groups + 2) * 2^-24 * C_abs; bf16 output adds half an ulp of bf16
(8 significant bits: at most 2^-8 relative), 2^-8 * (|C| + that bound).
"""

import numpy as np
import pytest
import torch

import oracle
import swiglu_backward_int8_amd as sq
from swiglu_backward_int8_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
G = 128
U = 2.0**-24


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sq.lib()


def operands(M, N, K, b_rows=1, seed=0, scale_range=(-6, 0)):
    rng = np.random.default_rng(seed)
    A = rng.integers(-127, 128, (M, K)).astype(np.int8)
    B = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sA = (rng.random((M, K // G)) * 10.0 ** rng.uniform(*scale_range, (M, K // G))).astype(np.float32)
    sB = (rng.random((-(-N // b_rows), K // G)) * 10.0 ** rng.uniform(*scale_range, (-(-N // b_rows), K // G)))
    return A, sA, B, sB.astype(np.float32)


def run_gpu(A, sA, B, sB, b_rows=1, out=torch.float32):
    M, N = A.shape[0], B.shape[0]
    t = [torch.from_numpy(a).to(DEV) for a in (A, sA, B, sB)]
    C = torch.full((M, N), float("nan"), dtype=out, device=DEV)  # every element must be written
    sq.i8_gemm_group_scaled(*t, C, b_rows_per_scale=b_rows)
    torch.cuda.synchronize()
    return C.float().cpu().numpy().astype(np.float64)


def check(got, want, want_abs, K, bf16=False, label=""):
    bound = (K // G + 2) * U * want_abs
    if bf16:
        bound = bound + 2.0**-8 * (np.abs(want) + bound) + 1e-45
    err = np.abs(got - want)
    bad = int((~(err <= bound)).sum())
    worst = float(np.nanmax(err / np.maximum(bound, 1e-300)))
    print("%s: %d of %d outside the bound, worst err/bound %.3g" % (label, bad, got.size, worst), flush=True)
    assert bad == 0


@pytest.mark.parametrize("M,N,K,b_rows", [(256, 256, 512, 1), (256, 256, 512, 128), (128, 128, 128, 1),
                                          (200, 136, 384, 1), (77, 300, 256, 128), (1, 1, 128, 1),
                                          (640, 384, 1024, 128), (33, 517, 640, 1)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_small_shapes(M, N, K, b_rows, out):
    A, sA, B, sB = operands(M, N, K, b_rows, seed=M * 7 + N + K)
    got = run_gpu(A, sA, B, sB, b_rows, torch.float32 if out == "f32" else torch.bfloat16)
    want, want_abs = oracle.i8_gemm_group_scaled(A, sA, B, sB, b_rows_per_scale=b_rows)
    check(got, want, want_abs, K, out == "bf16", "M=%d N=%d K=%d Bb=%d %s" % (M, N, K, b_rows, out))


def test_gemm_integer_extremes_exact():
    # unit scales and +-127 operands: every group sum is +-2,064,512 and the
    # totals (< 2^24) are exact in fp32
    M, N, K = 128, 256, 1024
    A = np.full((M, K), 127, np.int8)
    B = np.full((N, K), -127, np.int8)
    B[1::2] = 127
    ones = lambda r: np.ones((r, K // G), np.float32)
    got = run_gpu(A, ones(M), B, ones(N))
    want = (A[:1].astype(np.int64) @ B.astype(np.int64).T).astype(np.float64)
    assert np.array_equal(got, np.broadcast_to(want, got.shape))


def test_gemm_empty_contraction_writes_zeros():
    A = np.zeros((130, 0), np.int8)
    B = np.zeros((70, 0), np.int8)
    got = run_gpu(A, np.zeros((130, 0), np.float32), B, np.zeros((70, 0), np.float32))
    assert not got.any()


def test_gemm_wide_scale_range():
    # scales from 1e-30 to 1e10: fp32 products stay normal and the bound holds
    A, sA, B, sB = operands(128, 256, 512, seed=3, scale_range=(-15, 5))
    got = run_gpu(A, sA, B, sB)
    want, want_abs = oracle.i8_gemm_group_scaled(A, sA, B, sB)
    check(got, want, want_abs, 512, label="wide scales")


@pytest.mark.parametrize("use", ["dgrad", "wgrad"])
def test_gemm_full_size_sampled(use):
    # dgrad: M = T = 16384, N = D = 4096, K = 2H = 22016, block scales for the weight
    # wgrad: M = D = 4096, N = H = 11008, K = T = 16384, a scale per row of B (as y_s_t)
    M, N, K, b_rows = (16384, 4096, 22016, 128) if use == "dgrad" else (4096, 11008, 16384, 1)
    gen = torch.Generator(device=DEV).manual_seed(11 if use == "dgrad" else 12)
    A = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=DEV, generator=gen)
    B = torch.randint(-127, 128, (N, K), dtype=torch.int8, device=DEV, generator=gen)
    sA = torch.rand((M, K // G), device=DEV, generator=gen) * 1e-3
    sB = torch.rand((-(-N // b_rows), K // G), device=DEV, generator=gen) * 1e-2
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    print("case", use, M, N, K, flush=True)
    sq.i8_gemm_group_scaled(A, sA, B, sB, C, b_rows_per_scale=b_rows)
    torch.cuda.synchronize()
    assert not torch.isnan(C).any()
    rng = np.random.default_rng(5)
    rows = np.sort(np.concatenate([rng.choice(M, 40, replace=False), [0, M - 1]]))
    cols = np.sort(np.concatenate([rng.choice(N, 40, replace=False), [0, N - 1]]))
    An, sAn = A[rows].cpu().numpy(), sA[rows].cpu().numpy()
    Bn = B[cols].cpu().numpy()
    # the oracle with per-row B scales: expand the block scales of the sampled rows
    sBn = sB.cpu().numpy()[cols // b_rows]
    want, want_abs = oracle.i8_gemm_group_scaled(An, sAn, Bn, sBn)
    got = C[rows][:, cols].float().cpu().numpy().astype(np.float64)
    check(got, want, want_abs, K, bf16=True, label="%s sampled" % use)


def test_gemm_consumes_the_pass_outputs():
    # the fused pass on the GPU, then dgrad against a synthetic quantised weight
    x, dy = make_inputs("t4096_h1408", device=DEV, T=1024)
    T, H = dy.shape
    gq, gs, yq, ys = sq.empty_outputs(T, H, DEV)
    sq.silu_dot_fwd_bwd_quant_fuse(x, dy, gq, gs, yq, ys)
    D = 384
    gen = torch.Generator(device=DEV).manual_seed(21)
    W = torch.randint(-127, 128, (D, 2 * H), dtype=torch.int8, device=DEV, generator=gen)
    sW = torch.rand((D // 128, 2 * H // 128), device=DEV, generator=gen)
    C = torch.empty((T, D), dtype=torch.float32, device=DEV)
    sq.i8_gemm_group_scaled(gq, gs, W, sW, C, b_rows_per_scale=128)
    # wgrad: go_q_t [D, T] (synthetic) against y_q_t [H, T]
    go = torch.randint(-127, 128, (D, T), dtype=torch.int8, device=DEV, generator=gen)
    sgo = torch.rand((D, T // 128), device=DEV, generator=gen)
    C2 = torch.empty((D, H), dtype=torch.float32, device=DEV)
    sq.i8_gemm_group_scaled(go, sgo, yq, ys, C2, b_rows_per_scale=1)
    torch.cuda.synchronize()
    want, want_abs = oracle.i8_gemm_group_scaled(gq.cpu().numpy(), gs.cpu().numpy(), W.cpu().numpy(),
                                                 sW.cpu().numpy(), b_rows_per_scale=128)
    check(C.cpu().numpy().astype(np.float64), want, want_abs, 2 * H, label="dgrad of the pass")
    want, want_abs = oracle.i8_gemm_group_scaled(go.cpu().numpy(), sgo.cpu().numpy(), yq.cpu().numpy(),
                                                 ys.cpu().numpy())
    check(C2.cpu().numpy().astype(np.float64), want, want_abs, T, label="wgrad of the pass")


def test_gemm_binding_rejects_bad_tensors():
    A = torch.zeros((128, 256), dtype=torch.int8, device=DEV)
    s = torch.ones((128, 2), dtype=torch.float32, device=DEV)
    C = torch.empty((128, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        sq.i8_gemm_group_scaled(A.float(), s, A, s, C)
    with pytest.raises(ValueError):
        sq.i8_gemm_group_scaled(A, s, A, s, C.half())
    with pytest.raises(ValueError):
        sq.i8_gemm_group_scaled(A, s, A, s, C, b_rows_per_scale=64)
    with pytest.raises(ValueError):
        sq.i8_gemm_group_scaled(A[:, :200], s, A[:, :200], s, C)


# K groups of 64 and 32 (the pass's smaller group sizes): a stage of 128 of K
# holds two or four groups, each promoted on its own.
@pytest.mark.parametrize("group", [64, 32])
@pytest.mark.parametrize("M,N,K,b_rows", [(256, 256, 512, 1), (200, 136, 384, 128), (77, 300, 256, 1)])
def test_gemm_smaller_groups(group, M, N, K, b_rows):
    rng = np.random.default_rng(M + N + K + group)
    A = rng.integers(-127, 128, (M, K)).astype(np.int8)
    B = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sA = (rng.random((M, K // group)) * 10.0 ** rng.uniform(-6, 0, (M, K // group))).astype(np.float32)
    nb = -(-N // b_rows)
    sB = (rng.random((nb, K // group)) + 0.01).astype(np.float32)
    t = [torch.from_numpy(a).to(DEV) for a in (A, sA, B, sB)]
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    sq.i8_gemm_group_scaled(*t, C, b_rows_per_scale=b_rows, group_size=group)
    torch.cuda.synchronize()
    want, want_abs = oracle.i8_gemm_group_scaled(A, sA, B, sB, group_size=group, b_rows_per_scale=b_rows)
    check(C.cpu().numpy().astype(np.float64), want, want_abs, K * 128 // group,
          label="M=%d N=%d K=%d Bb=%d group=%d" % (M, N, K, b_rows, group))


@pytest.mark.parametrize("group", [64, 32])
def test_gemm_consumes_smaller_group_outputs(group):
    # the pass with group 64 or 32, then dgrad and wgrad with the same K groups
    x, dy = make_inputs("t4096_h1408", device=DEV, T=1024)
    T, H = dy.shape
    gq, gs, yq, ys = sq.empty_outputs(T, H, DEV, group=group)
    sq.silu_dot_fwd_bwd_quant_fuse(x, dy, gq, gs, yq, ys, group_size=group)
    D = 256
    gen = torch.Generator(device=DEV).manual_seed(23)
    W = torch.randint(-127, 128, (D, 2 * H), dtype=torch.int8, device=DEV, generator=gen)
    sW = torch.rand((D, 2 * H // group), device=DEV, generator=gen)
    C = torch.empty((T, D), dtype=torch.float32, device=DEV)
    sq.i8_gemm_group_scaled(gq, gs, W, sW, C, b_rows_per_scale=1, group_size=group)
    go = torch.randint(-127, 128, (D, T), dtype=torch.int8, device=DEV, generator=gen)
    sgo = torch.rand((D, T // group), device=DEV, generator=gen)
    C2 = torch.empty((D, H), dtype=torch.float32, device=DEV)
    sq.i8_gemm_group_scaled(go, sgo, yq, ys, C2, b_rows_per_scale=1, group_size=group)
    torch.cuda.synchronize()
    want, want_abs = oracle.i8_gemm_group_scaled(gq.cpu().numpy(), gs.cpu().numpy(), W.cpu().numpy(),
                                                 sW.cpu().numpy(), group_size=group)
    check(C.cpu().numpy().astype(np.float64), want, want_abs, 2 * H * 128 // group,
          label="dgrad of the pass, group %d" % group)
    want, want_abs = oracle.i8_gemm_group_scaled(go.cpu().numpy(), sgo.cpu().numpy(), yq.cpu().numpy(),
                                                 ys.cpu().numpy(), group_size=group)
    check(C2.cpu().numpy().astype(np.float64), want, want_abs, T * 128 // group,
          label="wgrad of the pass, group %d" % group)


# K a multiple of the group but not of 128: the last 128-wide stage holds one
# to three groups, and its missing chunks and scales read as zeros.
@pytest.mark.parametrize("M,N,K,group,b_rows", [(96, 130, 160, 32, 1), (128, 128, 192, 64, 1), (200, 70, 224, 32, 128),
                                                (256, 256, 32, 32, 1), (64, 300, 64, 64, 128), (33, 129, 96, 32, 1),
                                                (512, 384, 22080, 64, 128), (129, 257, 2144, 32, 1)])
def test_gemm_k_not_a_multiple_of_128(M, N, K, group, b_rows):
    rng = np.random.default_rng(M + 3 * N + K + group)
    A = rng.integers(-127, 128, (M, K)).astype(np.int8)
    B = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sA = (rng.random((M, K // group)) * 10.0 ** rng.uniform(-6, 0, (M, K // group))).astype(np.float32)
    sB = (rng.random((-(-N // b_rows), K // group)) + 0.01).astype(np.float32)
    t = [torch.from_numpy(a).to(DEV) for a in (A, sA, B, sB)]
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    sq.i8_gemm_group_scaled(*t, C, b_rows_per_scale=b_rows, group_size=group)
    torch.cuda.synchronize()
    want, want_abs = oracle.i8_gemm_group_scaled(A, sA, B, sB, group_size=group, b_rows_per_scale=b_rows)
    check(C.cpu().numpy().astype(np.float64), want, want_abs, (K // group) * G,
          label="M=%d N=%d K=%d Bb=%d group=%d" % (M, N, K, b_rows, group))


def test_gemm_consumes_straddling_pass_outputs():
    # H = 1056, group 64: a row group straddles d_gate and d_up, and dgrad's
    # K = 2H = 2112 ends half way into a 128-wide stage
    from swiglu_backward_int8_amd.inputs import random_inputs
    T, H, group, D = 256, 1056, 64, 192
    x, dy = random_inputs(T, H, device=DEV, seed=31)
    gq, gs, yq, ys = sq.empty_outputs(T, H, DEV, group=group)
    sq.silu_dot_fwd_bwd_quant_fuse(x, dy, gq, gs, yq, ys, group_size=group)
    gen = torch.Generator(device=DEV).manual_seed(29)
    W = torch.randint(-127, 128, (D, 2 * H), dtype=torch.int8, device=DEV, generator=gen)
    sW = torch.rand((D, 2 * H // group), device=DEV, generator=gen)
    C = torch.empty((T, D), dtype=torch.float32, device=DEV)
    sq.i8_gemm_group_scaled(gq, gs, W, sW, C, b_rows_per_scale=1, group_size=group)
    torch.cuda.synchronize()
    want, want_abs = oracle.i8_gemm_group_scaled(gq.cpu().numpy(), gs.cpu().numpy(), W.cpu().numpy(),
                                                 sW.cpu().numpy(), group_size=group)
    check(C.cpu().numpy().astype(np.float64), want, want_abs, (2 * H // group) * G,
          label="dgrad of the straddling pass")
