"""Python binding for libsiluquant (fused SwiGLU backward + two-axis int8 quantisation).

Argument marshalling only: every step of the pass runs in the HIP kernel inside
``libsiluquant.so``; PyTorch supplies device memory and the current stream.
The binding has the name and argument order of the entry point listed on the
page "kernelgen-challenge-9-task3-silu-quant" (githubhelp.com).  If the built
library is missing the call raises; there is no other implementation behind it.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsiluquant.so")
GROUP = 128
GROUPS = (32, 64, 128)  # group sizes of the backward pass (they divide its 128 x 128 tiles)

SILUQUANT_OK = 0
_ERRORS = {
    1: (ValueError, "NULL_PTR"),
    2: (ValueError, "BAD_SHAPE"),
    3: (ValueError, "BAD_GROUP"),
    4: (ValueError, "MISALIGNED"),
    5: (ValueError, "OVERLAP"),
    6: (RuntimeError, "DEVICE"),
    7: (RuntimeError, "LAUNCH_FAILED"),
}

EXPORTED = ("silu_dot_fwd_bwd_quant_fuse", "silu_dot_fwd_bwd_quant_fuse_fp8", "silu_fwd_quant", "silu_fwd_quant_q8_1",
            "kquant_swiglu_q8_1_rows", "i8_gemm_group_scaled", "siluquant_prepare", "siluquant_strerror", "siluquant_algorithmic_bytes",
            "siluquant_eval_sigmoid", "siluquant_eval_intermediates")

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libsiluquant.so is not built (run swiglu_backward_int8_amd/_build.py or "
                               "__graft_entry__.build()); there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        L.silu_dot_fwd_bwd_quant_fuse.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp]
        L.silu_dot_fwd_bwd_quant_fuse.restype = ctypes.c_int
        L.silu_dot_fwd_bwd_quant_fuse_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp]
        L.silu_dot_fwd_bwd_quant_fuse_fp8.restype = ctypes.c_int
        L.siluquant_prepare.argtypes = []
        L.siluquant_prepare.restype = ctypes.c_int
        L.siluquant_strerror.argtypes = [ctypes.c_int]
        L.siluquant_strerror.restype = ctypes.c_char_p
        L.siluquant_algorithmic_bytes.argtypes = [i64, i64, i64]
        L.siluquant_algorithmic_bytes.restype = i64
        L.silu_fwd_quant.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
        L.silu_fwd_quant.restype = ctypes.c_int
        L.silu_fwd_quant_q8_1.argtypes = [vp, vp, vp, i64, i64, vp]
        L.silu_fwd_quant_q8_1.restype = ctypes.c_int
        L.kquant_swiglu_q8_1_rows.argtypes = [vp, vp, vp, vp, vp, i64, i64, vp]
        L.kquant_swiglu_q8_1_rows.restype = ctypes.c_int
        L.i8_gemm_group_scaled.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int, vp]
        L.i8_gemm_group_scaled.restype = ctypes.c_int
        L.siluquant_eval_sigmoid.argtypes = [vp, vp, i64, vp]
        L.siluquant_eval_sigmoid.restype = ctypes.c_int
        L.siluquant_eval_intermediates.argtypes = [vp, vp, vp, vp, i64, i64, vp]
        L.siluquant_eval_intermediates.restype = ctypes.c_int
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().siluquant_strerror(int(code)).decode()


def algorithmic_bytes(T: int, H: int, group: int = GROUP) -> int:
    """Bytes one call must move (reads + writes), as the library counts them."""
    return int(lib().siluquant_algorithmic_bytes(int(T), int(H), int(group)))


def _check(code: int, what: str):
    if code != SILUQUANT_OK:
        exc, name = _ERRORS.get(code, (RuntimeError, "UNKNOWN"))
        raise exc("%s failed: %s (%s)" % (what, name, strerror(code)))


def output_shapes(T: int, H: int, group: int = GROUP) -> dict:
    """Shapes of (grad_input_q, grad_input_s, y_q_t, y_s_t); the last token group
    of a T that is not a multiple of 128 is shorter."""
    return {
        "grad_input_q": (T, 2 * H),
        "grad_input_s": (T, -(-2 * H // group)),
        "y_q_t": (H, T),
        "y_s_t": (H, -(-T // group)),
    }


def raw_call(x_ptr: int, grad_y_ptr: int, gq_ptr: int, gs_ptr: int, yq_ptr: int, ys_ptr: int, T: int, H: int,
             group: int, stream: int, fp8: bool = False) -> int:
    """The C entry point (int8, or E4M3 with fp8=True) with plain integers for
    pointers; returns the status code."""
    fn = lib().silu_dot_fwd_bwd_quant_fuse_fp8 if fp8 else lib().silu_dot_fwd_bwd_quant_fuse
    return int(fn(x_ptr, grad_y_ptr, gq_ptr, gs_ptr, yq_ptr, ys_ptr, int(T), int(H), int(group), stream))


def silu_dot_fwd_bwd_quant_fuse(x, grad_y, grad_input_q, grad_input_s, y_q_t, y_s_t, group_size: int = GROUP):
    """Recompute y = silu(gate) * up from x = [gate | up] and write the int8 codes
    and fp32 scales of [d_gate, d_up] (per row, groups of group_size channels)
    and of y^T (groups of group_size tokens) into the given output tensors.
    group_size is 128 (the default), 64 or 32; any H: when it is not a multiple
    of group_size one group straddles d_gate and d_up, and when it is not a
    multiple of 8 (rows off 16 bytes) a slower tiled path runs.
    Enqueued on the current stream of x's device; returns None."""
    _backward(x, grad_y, grad_input_q, grad_input_s, y_q_t, y_s_t, group_size, fp8=False)


def silu_dot_fwd_bwd_quant_fuse_fp8(x, grad_y, grad_input_q, grad_input_s, y_q_t, y_s_t, group_size: int = GROUP):
    """The same pass with OCP FP8 E4M3 codes (scale = amax / 448).  The code
    tensors are uint8 (the E4M3 bit patterns) or torch.float8_e4m3fn."""
    _backward(x, grad_y, grad_input_q, grad_input_s, y_q_t, y_s_t, group_size, fp8=True)


def bind_backward(x, grad_y, grad_input_q, grad_input_s, y_q_t, y_s_t, group_size: int = GROUP, fp8: bool = False):
    """Check the six tensors once, as silu_dot_fwd_bwd_quant_fuse(_fp8) does,
    and return a function of no arguments that enqueues the pass on them (on
    the current stream of x's device at each call) without checking them
    again: for loops that run the pass many times on the same buffers, where
    the checks would otherwise cost host time on every call.  The function
    holds the tensors; they must not be resized while it is in use."""
    import torch

    T, H = _validate_backward(x, grad_y, grad_input_q, grad_input_s, y_q_t, y_s_t, group_size, fp8)
    dev = x.device
    tensors = (x, grad_y, grad_input_q, grad_input_s, y_q_t, y_s_t)
    ptrs = tuple(t.data_ptr() for t in tensors)
    what = "silu_dot_fwd_bwd_quant_fuse_fp8" if fp8 else "silu_dot_fwd_bwd_quant_fuse"

    def run():
        with torch.cuda.device(dev):
            code = raw_call(*ptrs, T, H, group_size, torch.cuda.current_stream(dev).cuda_stream, fp8=fp8)
        _check(code, what)

    run.tensors = tensors
    return run


def _backward(x, grad_y, grad_input_q, grad_input_s, y_q_t, y_s_t, group_size: int, fp8: bool):
    import torch

    T, H = _validate_backward(x, grad_y, grad_input_q, grad_input_s, y_q_t, y_s_t, group_size, fp8)
    dev = x.device
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        code = raw_call(x.data_ptr(), grad_y.data_ptr(), grad_input_q.data_ptr(), grad_input_s.data_ptr(),
                        y_q_t.data_ptr(), y_s_t.data_ptr(), T, H, group_size, stream, fp8=fp8)
    _check(code, "silu_dot_fwd_bwd_quant_fuse_fp8" if fp8 else "silu_dot_fwd_bwd_quant_fuse")


def _validate_backward(x, grad_y, grad_input_q, grad_input_s, y_q_t, y_s_t, group_size: int, fp8: bool):
    """The binding's checks of the pass's tensors; returns (T, H)."""
    import torch

    code_types = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8)) if fp8 else (torch.int8,)
    if x.dim() != 2 or grad_y.dim() != 2 or tuple(x.shape) != (grad_y.shape[0], 2 * grad_y.shape[1]):
        raise ValueError("x must be [T, 2H] and grad_y [T, H]; got %s and %s" % (tuple(x.shape), tuple(grad_y.shape)))
    T, H = int(grad_y.shape[0]), int(grad_y.shape[1])
    if group_size not in GROUPS:
        raise ValueError("group_size must be one of %s" % (GROUPS,))
    want = output_shapes(T, H, group_size)
    checks = [
        ("x", x, torch.bfloat16, (T, 2 * H)),
        ("grad_y", grad_y, torch.bfloat16, (T, H)),
        ("grad_input_q", grad_input_q, code_types, want["grad_input_q"]),
        ("grad_input_s", grad_input_s, torch.float32, want["grad_input_s"]),
        ("y_q_t", y_q_t, code_types, want["y_q_t"]),
        ("y_s_t", y_s_t, torch.float32, want["y_s_t"]),
    ]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU; got %s" % dev)
    for name, t, dt, shape in checks:
        if t.dtype not in (dt if isinstance(dt, tuple) else (dt,)):
            raise ValueError("%s must be %s, got %s" % (name, dt, t.dtype))
        if t.device != dev:
            raise ValueError("%s is on %s, x on %s" % (name, t.device, dev))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if tuple(t.shape) != tuple(shape):
            raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return T, H


def silu_fwd_quant(x, y_q, y_s, row_weight=None, y_bf16=None, group_size: int = GROUP):
    """Forward SwiGLU with row-wise int8 quantisation: y = bf16((silu(gate) * up)
    * row_weight[t]) from x = [gate | up] [T, 2H]; writes y_q int8 [T, H] and
    y_s fp32 [T, ceil(H/group_size)] (group_size 128, 64 or 32; any H, the last
    group of a row partial when H is not a multiple of group_size),
    and y_bf16 [T, H] if given.  Enqueued on the current stream of x's device;
    returns None."""
    import torch

    if x.dim() != 2 or x.shape[1] % 2:
        raise ValueError("x must be [T, 2H]")
    T, H = int(x.shape[0]), int(x.shape[1]) // 2
    if group_size not in GROUPS:
        raise ValueError("group_size must be one of %s" % (GROUPS,))
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU; got %s" % dev)
    checks = [("x", x, torch.bfloat16, (T, 2 * H)), ("y_q", y_q, torch.int8, (T, H)),
              ("y_s", y_s, torch.float32, (T, -(-H // group_size)))]
    if row_weight is not None:
        checks.append(("row_weight", row_weight, torch.float32, (T,)))
    if y_bf16 is not None:
        checks.append(("y_bf16", y_bf16, torch.bfloat16, (T, H)))
    for name, t, dt, shape in checks:
        if t.dtype != dt or t.device != dev or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
            raise ValueError("%s must be a contiguous %s tensor of shape %s on %s" % (name, dt, shape, dev))
    with torch.cuda.device(dev):
        code = int(lib().silu_fwd_quant(x.data_ptr(), row_weight.data_ptr() if row_weight is not None else None,
                                        y_q.data_ptr(), y_s.data_ptr(),
                                        y_bf16.data_ptr() if y_bf16 is not None else None, T, H, group_size,
                                        torch.cuda.current_stream(dev).cuda_stream))
    _check(code, "silu_fwd_quant")


Q8_1_BLOCK = 36  # bytes per 32 channels: binary16 d and sum, then 32 int8 codes


def silu_fwd_quant_q8_1(x, y_q8, row_weight=None):
    """Forward SwiGLU quantised in the q8_1 block layout: y = bf16((silu(gate)
    * up) * row_weight[t]) from x = [gate | up] [T, 2H] (H a multiple of 32)
    into y_q8 uint8 [T, (H/32) * 36]: per 32 channels the binary16 d (the
    group scale, amax / 127) and sum (fl32(d * sum of the codes)), then the
    32 int8 codes.  Enqueued on the current stream of x's device; returns None."""
    import torch

    if x.dim() != 2 or x.shape[1] % 2:
        raise ValueError("x must be [T, 2H]")
    T, H = int(x.shape[0]), int(x.shape[1]) // 2
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU; got %s" % dev)
    checks = [("x", x, torch.bfloat16, (T, 2 * H)), ("y_q8", y_q8, torch.uint8, (T, (H // 32) * Q8_1_BLOCK))]
    if row_weight is not None:
        checks.append(("row_weight", row_weight, torch.float32, (T,)))
    for name, t, dt, shape in checks:
        if t.dtype != dt or t.device != dev or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
            raise ValueError("%s must be a contiguous %s tensor of shape %s on %s" % (name, dt, shape, dev))
    with torch.cuda.device(dev):
        code = int(lib().silu_fwd_quant_q8_1(x.data_ptr(), row_weight.data_ptr() if row_weight is not None else None,
                                             y_q8.data_ptr(), T, H, torch.cuda.current_stream(dev).cuda_stream))
    _check(code, "silu_fwd_quant_q8_1")


def kquant_swiglu_q8_1_rows(gate, up, out_q8, w=None, h_bf16=None):
    """The page's fused launch shape (kquant_swiglu_q8_1_rows): separate bf16
    gate and up [rows, inter] (inter a multiple of 32), optional fp32 weight
    per row; writes the q8_1 blocks of h = bf16((silu(gate) * up) * w[row])
    into out_q8 uint8 [rows, (inter/32) * 36] and, if given, h into h_bf16
    [rows, inter].  Enqueued on the current stream of gate's device; returns
    None."""
    import torch

    if gate.dim() != 2:
        raise ValueError("gate must be [rows, inter]")
    rows, inter = int(gate.shape[0]), int(gate.shape[1])
    dev = gate.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU; got %s" % dev)
    checks = [("gate", gate, torch.bfloat16, (rows, inter)), ("up", up, torch.bfloat16, (rows, inter)),
              ("out_q8", out_q8, torch.uint8, (rows, (inter // 32) * Q8_1_BLOCK))]
    if w is not None:
        checks.append(("w", w, torch.float32, (rows,)))
    if h_bf16 is not None:
        checks.append(("h_bf16", h_bf16, torch.bfloat16, (rows, inter)))
    for name, t, dt, shape in checks:
        if t.dtype != dt or t.device != dev or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
            raise ValueError("%s must be a contiguous %s tensor of shape %s on %s" % (name, dt, shape, dev))
    with torch.cuda.device(dev):
        code = int(lib().kquant_swiglu_q8_1_rows(gate.data_ptr(), up.data_ptr(),
                                                 w.data_ptr() if w is not None else None,
                                                 h_bf16.data_ptr() if h_bf16 is not None else None,
                                                 out_q8.data_ptr(), rows, inter,
                                                 torch.cuda.current_stream(dev).cuda_stream))
    _check(code, "kquant_swiglu_q8_1_rows")


def forward_q8_1_bytes(T: int, H: int, with_weight: bool = False) -> int:
    """Bytes the q8_1 forward quantiser must move: x (4 per pair) in, 36 per
    32 channels out, plus the row weights."""
    return 4 * T * H + T * (H // 32) * Q8_1_BLOCK + (4 * T if with_weight else 0)


GEMM_OUT_F32, GEMM_OUT_BF16 = 0, 1


def i8_gemm_group_scaled(A, sA, B, sB, C, b_rows_per_scale: int = 1, group_size: int = GROUP):
    """C = A . B^T of group-scaled int8 operands on the matrix cores:
    C[m, n] = sum_g sA[m, g] * sB[n // b_rows_per_scale, g] * (A[m, group g] . B[n, group g]).
    Groups are group_size (128, 64 or 32) wide along K; K is a multiple of it.
    A int8 [M, K], sA fp32 [M, K/group_size], B int8 [N, K], sB fp32
    [ceil(N / b_rows_per_scale), K/group_size] (b_rows_per_scale 1 or 128); C
    fp32 or bf16 [M, N] is overwritten.  Enqueued on the current stream of A's
    device."""
    import torch

    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[1]:
        raise ValueError("A must be [M, K] and B [N, K]")
    M, K = int(A.shape[0]), int(A.shape[1])
    N = int(B.shape[0])
    if group_size not in GROUPS or K % group_size:
        raise ValueError("group_size must be one of %s and K a multiple of it" % (GROUPS,))
    if b_rows_per_scale not in (1, 128):
        raise ValueError("b_rows_per_scale must be 1 or 128")
    dev = A.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU; got %s" % dev)
    groups = K // group_size
    if C.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("C must be float32 or bfloat16")
    checks = [("A", A, torch.int8, (M, K)), ("sA", sA, torch.float32, (M, groups)),
              ("B", B, torch.int8, (N, K)), ("sB", sB, torch.float32, (-(-N // b_rows_per_scale), groups)),
              ("C", C, C.dtype, (M, N))]
    for name, t, dt, shape in checks:
        if t.dtype != dt or t.device != dev or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
            raise ValueError("%s must be a contiguous %s tensor of shape %s on %s" % (name, dt, shape, dev))
    out = GEMM_OUT_F32 if C.dtype == torch.float32 else GEMM_OUT_BF16
    with torch.cuda.device(dev):
        code = int(lib().i8_gemm_group_scaled(A.data_ptr(), sA.data_ptr(), B.data_ptr(), sB.data_ptr(),
                                              C.data_ptr(), M, N, K, group_size, b_rows_per_scale, out,
                                              torch.cuda.current_stream(dev).cuda_stream))
    _check(code, "i8_gemm_group_scaled")


def forward_bytes(T: int, H: int, with_bf16: bool = False, with_weight: bool = False, group: int = GROUP) -> int:
    """Bytes the forward quantiser must move: x (4 per pair) in, codes (1) and
    one fp32 scale per `group` codes out, plus bf16 y (2) and the row weights."""
    return 5 * T * H + 4 * T * (-(-H // group)) + (2 * T * H if with_bf16 else 0) + (4 * T if with_weight else 0)


def empty_outputs(T: int, H: int, device, group: int = GROUP, fp8: bool = False):
    """Freshly allocated (grad_input_q, grad_input_s, y_q_t, y_s_t) for a call
    (uint8 code tensors with fp8=True)."""
    import torch

    s = output_shapes(T, H, group)
    code = torch.uint8 if fp8 else torch.int8
    return (torch.empty(s["grad_input_q"], dtype=code, device=device),
            torch.empty(s["grad_input_s"], dtype=torch.float32, device=device),
            torch.empty(s["y_q_t"], dtype=code, device=device),
            torch.empty(s["y_s_t"], dtype=torch.float32, device=device))


def prepare():
    """Build the sigmoid table on the current device now (the first call does it otherwise)."""
    _check(int(lib().siluquant_prepare()), "siluquant_prepare")


def eval_sigmoid(gate):
    """Diagnostic: the kernel's sigmoid of each bf16 gate (a 1-D CUDA bf16 tensor)."""
    import torch

    if gate.dtype != torch.bfloat16 or gate.device.type != "cuda" or not gate.is_contiguous():
        raise ValueError("gate must be a contiguous bf16 GPU tensor")
    out = torch.empty(gate.shape, dtype=torch.float32, device=gate.device)
    with torch.cuda.device(gate.device):
        code = lib().siluquant_eval_sigmoid(gate.data_ptr(), out.data_ptr(), gate.numel(),
                                            torch.cuda.current_stream(gate.device).cuda_stream)
    _check(code, "siluquant_eval_sigmoid")
    return out


def eval_intermediates(x, grad_y):
    """Diagnostic: bf16 y [T, H] and [d_gate | d_up] [T, 2H] as the kernel computes them."""
    import torch

    T, H = grad_y.shape
    for name, t in (("x", x), ("grad_y", grad_y)):
        if t.dtype != torch.bfloat16 or t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError("%s must be a contiguous bf16 GPU tensor" % name)
    if tuple(x.shape) != (T, 2 * H):
        raise ValueError("x must be [T, 2H]")
    y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    d = torch.empty((T, 2 * H), dtype=torch.bfloat16, device=x.device)
    with torch.cuda.device(x.device):
        code = lib().siluquant_eval_intermediates(x.data_ptr(), grad_y.data_ptr(), y.data_ptr(), d.data_ptr(),
                                                  T, H, torch.cuda.current_stream(x.device).cuda_stream)
    _check(code, "siluquant_eval_intermediates")
    return y, d
