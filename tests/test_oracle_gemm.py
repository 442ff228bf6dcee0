"""Pins for the oracle's group-scaled int8 product (CPU only).

C = A . B^T with A [M, K], B [N, K] int8 and one fp32 scale per row and
128-wide group of K (B's scale rows optionally shared by 128-row blocks).
Pinned by:

* unit scales: C is the plain integer product, compared with numpy's int64
  matmul exactly (including all-+-127 operands over a long K);
* a hand-worked two-group example whose value follows from the definition
  without running any float code;
* the dequantised-operand form: (sA (x) A) . (sB (x) B)^T by numpy's float64
  matmul, a different evaluation of the same quantity, within fp64 rounding;
* block scales equal per-row scales repeated over each 128-row block;
* exact scaling by powers of two and the transpose symmetry
  C(A, sA, B, sB) = C(B, sB, A, sA)^T;
* consumption of the pass's own layouts: the product of grad_input_q with a
  quantised weight, and of a quantised gradient with y_q_t, lies within the
  quantisation error bound of the unquantised bf16 product.
"""

import numpy as np
import pytest
import torch

import oracle
from swiglu_backward_int8_amd.inputs import random_inputs

G = 128


def _rand(rng, M, N, K, b_rows=1):
    A = rng.integers(-127, 128, (M, K)).astype(np.int8)
    B = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sA = (rng.random((M, K // G)) * 10.0 ** rng.uniform(-6, 0, (M, K // G))).astype(np.float32)
    sB = (rng.random((-(-N // b_rows), K // G)) + 0.01).astype(np.float32)
    return A, sA, B, sB


def test_unit_scales_are_the_integer_product():
    rng = np.random.default_rng(1)
    A = rng.integers(-127, 128, (7, 512)).astype(np.int8)
    B = rng.integers(-127, 128, (5, 512)).astype(np.int8)
    C, C_abs = oracle.i8_gemm_group_scaled(A, np.ones((7, 4), np.float32), B, np.ones((5, 4), np.float32))
    want = A.astype(np.int64) @ B.astype(np.int64).T
    assert np.array_equal(C, want.astype(np.float64))
    # extremes: 127 * 127 * 4096 = 66,064,384 per entry, exact in int64 and double
    A = np.full((2, 4096), 127, np.int8)
    B = np.full((3, 4096), -127, np.int8)
    C, C_abs = oracle.i8_gemm_group_scaled(A, np.ones((2, 32), np.float32), B, np.ones((3, 32), np.float32))
    assert np.all(C == -66_064_384.0) and np.all(C_abs == 66_064_384.0)


def test_worked_example_two_groups():
    # group 0: 128 * (1 * 3) = 384, times 0.5 * 2 -> 384
    # group 1: 128 * (2 * -1) = -256, times 0.25 * 4 -> -256
    A = np.array([[1] * 128 + [2] * 128], np.int8)
    B = np.array([[3] * 128 + [-1] * 128], np.int8)
    C, C_abs = oracle.i8_gemm_group_scaled(A, np.array([[0.5, 0.25]], np.float32), B,
                                           np.array([[2.0, 4.0]], np.float32))
    assert C[0, 0] == 128.0 and C_abs[0, 0] == 640.0


def test_dequantised_operand_form():
    rng = np.random.default_rng(2)
    for M, N, K, b_rows in ((9, 11, 384, 1), (4, 300, 256, 128), (1, 1, 128, 1)):
        A, sA, B, sB = _rand(rng, M, N, K, b_rows)
        C, C_abs = oracle.i8_gemm_group_scaled(A, sA, B, sB, b_rows_per_scale=b_rows)
        Ad = A.astype(np.float64) * np.repeat(sA.astype(np.float64), G, axis=1)
        sBr = np.repeat(sB.astype(np.float64), b_rows, axis=0)[:N]
        Bd = B.astype(np.float64) * np.repeat(sBr, G, axis=1)
        want = Ad @ Bd.T
        assert np.all(np.abs(C - want) <= 1e-13 * C_abs + 1e-300)


def test_block_scales_equal_repeated_row_scales():
    rng = np.random.default_rng(3)
    A, sA, B, sB = _rand(rng, 6, 300, 256, 128)
    C1, _ = oracle.i8_gemm_group_scaled(A, sA, B, sB, b_rows_per_scale=128)
    C2, _ = oracle.i8_gemm_group_scaled(A, sA, B, np.repeat(sB, 128, axis=0)[:300], b_rows_per_scale=1)
    assert np.array_equal(C1, C2)


def test_power_of_two_scaling_and_transpose_symmetry():
    rng = np.random.default_rng(4)
    A, sA, B, sB = _rand(rng, 8, 6, 384)
    C, _ = oracle.i8_gemm_group_scaled(A, sA, B, sB)
    C2, _ = oracle.i8_gemm_group_scaled(A, sA * np.float32(4), B, sB)
    assert np.array_equal(C2, 4 * C)
    Ct, _ = oracle.i8_gemm_group_scaled(B, sB, A, sA)
    assert np.array_equal(Ct, C.T)


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _quant_rows(W):
    """Row-wise 128-group int8 quantisation of a float matrix with the oracle's
    group quantiser (the weight side of a product)."""
    N, K = W.shape
    q = np.zeros((N, K), np.int8)
    s = np.zeros((N, K // G), np.float32)
    for n in range(N):
        for g in range(K // G):
            q[n, g * G:(g + 1) * G], s[n, g] = oracle.quant_group(W[n, g * G:(g + 1) * G])
    return q, s


def test_consumes_the_pass_layouts():
    T, H, D = 256, 128, 64
    x, dy = random_inputs(T, H, seed=9)
    gq, gs, yq, ys = oracle.silu_dot_fwd_bwd_quant_fuse(_bits(x), _bits(dy))
    Y, Dg = oracle.intermediates(_bits(x), _bits(dy))
    rng = np.random.default_rng(5)
    # dgrad: [T, 2H] . W[D, 2H]^T, K = 2H carries grad_input_q's row groups
    W = rng.standard_normal((D, 2 * H)).astype(np.float32)
    wq, ws = _quant_rows(W)
    C, _ = oracle.i8_gemm_group_scaled(gq, gs, wq, ws)
    Dd = gq.astype(np.float64) * np.repeat(gs, G, axis=1)
    Wd = wq.astype(np.float64) * np.repeat(ws, G, axis=1)
    exact = Dg.astype(np.float64) @ W.astype(np.float64).T
    # |D Wd - Dq Wdq| <= |D - Dq| |Wd| + |D| |W - Wdq|, each error at most half a step
    err_d = np.repeat(gs.astype(np.float64), G, axis=1) * 0.5 * (1 + 2.0**-15)
    err_w = np.repeat(ws.astype(np.float64), G, axis=1) * 0.5 * (1 + 2.0**-15)
    bound = err_d @ np.abs(Wd).T + np.abs(Dg.astype(np.float64)) @ err_w.T
    assert np.all(np.abs(C - exact) <= bound * (1 + 1e-9) + 1e-30)
    assert np.abs(C - Dd @ Wd.T).max() <= 1e-12 * np.abs(C).max()
    # wgrad of the down projection: dW[D, H] = go^T [D, T] . y [T, H], K = T
    # carries y_q_t's token groups (B = y_q_t [H, T], one scale per row and group)
    go = rng.standard_normal((T, D)).astype(np.float32)
    aq, as_ = _quant_rows(np.ascontiguousarray(go.T))
    C, _ = oracle.i8_gemm_group_scaled(aq, as_, yq, ys)
    exact = go.T.astype(np.float64) @ Y.astype(np.float64)
    err_a = np.repeat(as_.astype(np.float64), G, axis=1) * 0.5 * (1 + 2.0**-15)
    err_y = np.repeat(ys.astype(np.float64), G, axis=1) * 0.5 * (1 + 2.0**-15)
    Ad = aq.astype(np.float64) * np.repeat(as_, G, axis=1)
    bound = err_a @ np.abs(Y.astype(np.float64)) + np.abs(Ad) @ err_y.T
    assert np.all(np.abs(C - exact) <= bound * (1 + 1e-9) + 1e-30)


def test_rejects_bad_shapes():
    A = np.zeros((2, 200), np.int8)
    with pytest.raises(ValueError):
        oracle.i8_gemm_group_scaled(A, np.ones((2, 2), np.float32), A, np.ones((2, 2), np.float32))
