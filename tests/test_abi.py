"""The C-ABI library: it loads, exports every entry point its header declares,
and rejects bad arguments before touching any device (CPU only)."""

import ctypes
import os
import re

import pytest

import swiglu_backward_int8_amd as sq
from swiglu_backward_int8_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "siluquant.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sq.LIB_PATH):
        _build.build()
    return sq.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    assert "silu_dot_fwd_bwd_quant_fuse" in names
    assert set(names) == set(sq.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_product_library_does_not_link_the_oracle():
    import subprocess

    out = subprocess.run(["nm", "-D", sq.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "oracle" not in out
    deps = subprocess.run(["readelf", "-d", sq.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "liboracle" not in deps


def test_library_allocates_nothing_and_never_waits():
    # The boundary enqueues kernels on the caller's stream and returns: the
    # library imports no HIP routine that allocates or frees memory, creates
    # or destroys a stream or event, copies memory or waits for the device.
    import subprocess

    out = subprocess.run(["nm", "-D", "--undefined-only", sq.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    names = [line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()]
    hip = sorted({n for n in names if n.startswith("hip")})
    allowed = {"hipDeviceGetAttribute", "hipFuncGetAttributes", "hipGetDevice", "hipGetLastError",
               "hipLaunchKernel"}
    assert hip and set(hip) <= allowed, hip
    assert "__hipRegisterFatBinary" in out  # the kernels' code object, registered at load


# Fake, well-aligned, non-overlapping addresses: every call below must be
# rejected by the host-side checks, so none of them is ever dereferenced.
BASE = 1 << 40


def _ptrs(T, H, misalign=None, null=None, overlap=False):
    sizes = [4 * T * H, 2 * T * H, 2 * T * H, 4 * T * -(-2 * H // 128), T * H, 4 * H * -(-T // 128)]
    ptrs, at = [], BASE
    for s in sizes:
        ptrs.append(at)
        at += ((max(s, 1) + 4095) // 4096) * 4096
    if misalign is not None:
        ptrs[misalign] += 2
    if null is not None:
        ptrs[null] = 0
    if overlap:
        ptrs[4] = ptrs[2] + 64  # y_q_t inside grad_input_q
    return ptrs


@pytest.mark.parametrize("T,H,group,code", [
    (256, 256, 48, 3), (256, 256, 0, 3), (256, 256, 256, 3), (256, 256, 16, 3),
    (-128, 256, 128, 2), (256, -128, 128, 2), (-1, 100, 64, 2), (100, -68, 32, 2),
    (256, (1 << 22) + 8, 128, 2), (256, (1 << 22) + 3, 64, 2), ((1 << 23) + 1, 8, 32, 2), ((1 << 23) + 1, 5, 128, 2),
])
@pytest.mark.parametrize("fp8", [False, True])
def test_bad_shape_and_group(lib, T, H, group, code, fp8):
    assert sq.raw_call(*_ptrs(abs(T), abs(H)), T, H, group, 0, fp8=fp8) == code


@pytest.mark.parametrize("which", range(6))
@pytest.mark.parametrize("fp8", [False, True])
def test_null_pointer(lib, which, fp8):
    assert sq.raw_call(*_ptrs(256, 256, null=which), 256, 256, 128, 0, fp8=fp8) == 1


@pytest.mark.parametrize("which", range(6))
@pytest.mark.parametrize("fp8", [False, True])
def test_misaligned(lib, which, fp8):
    assert sq.raw_call(*_ptrs(256, 256, misalign=which), 256, 256, 128, 0, fp8=fp8) == 4


@pytest.mark.parametrize("fp8", [False, True])
def test_overlap(lib, fp8):
    assert sq.raw_call(*_ptrs(256, 256, overlap=True), 256, 256, 128, 0, fp8=fp8) == 5
    p = _ptrs(256, 256)
    p[1] = p[0]  # grad_y aliases x
    assert sq.raw_call(*p, 256, 256, 128, 0, fp8=fp8) == 5


@pytest.mark.parametrize("fp8", [False, True])
def test_empty_is_a_no_op(lib, fp8):
    # nothing to do: success without any pointer being looked at
    assert sq.raw_call(0, 0, 0, 0, 0, 0, 0, 256, 128, 0, fp8=fp8) == 0
    assert sq.raw_call(0, 0, 0, 0, 0, 0, 256, 0, 128, 0, fp8=fp8) == 0


def test_diagnostics_reject_bad_arguments(lib):
    assert lib.siluquant_eval_sigmoid(None, None, -1, None) == 2
    assert lib.siluquant_eval_sigmoid(None, None, 0, None) == 0
    assert lib.siluquant_eval_sigmoid(None, BASE, 10, None) == 1
    assert lib.siluquant_eval_sigmoid(BASE + 1, BASE + 4096, 10, None) == 4
    assert lib.siluquant_eval_sigmoid(BASE, BASE + 8, 10, None) == 5
    assert lib.siluquant_eval_intermediates(None, None, None, None, 128, -1, None) == 2
    assert lib.siluquant_eval_intermediates(BASE, None, BASE, BASE, 128, 128, None) == 1


def test_strerror(lib):
    for code in range(8):
        assert sq.strerror(code)
    assert sq.strerror(99) == "unknown status"


# Algorithmic bytes per call: reads x (4 B) and grad_y (2 B) per (t, h) pair,
# writes 2 + 1 code bytes and one fp32 scale per 128 codes on each axis.
# Totals counted tensor by tensor for the five workloads.
BYTES = {
    (256, 256): 262_144 + 131_072 + 131_072 + 4_096 + 65_536 + 2_048,
    (4096, 1408): 23_068_672 + 11_534_336 + 11_534_336 + 360_448 + 5_767_168 + 180_224,
    (8192, 4096): 134_217_728 + 67_108_864 + 67_108_864 + 2_097_152 + 33_554_432 + 1_048_576,
    (16384, 11008): 721_420_288 + 360_710_144 + 360_710_144 + 11_272_192 + 180_355_072 + 5_636_096,
    (32768, 2048): 268_435_456 + 134_217_728 + 134_217_728 + 4_194_304 + 67_108_864 + 2_097_152,
}


def test_algorithmic_bytes_ragged_tokens(lib):
    # T = 200: 2 token groups (128 + 72), 2H/128 = 4 row groups
    T, H = 200, 256
    assert sq.algorithmic_bytes(T, H) == 9 * T * H + 4 * T * 4 + 4 * H * 2


@pytest.mark.parametrize("shape", sorted(BYTES))
def test_algorithmic_bytes(lib, shape):
    assert sq.algorithmic_bytes(*shape) == BYTES[shape]
    assert BYTES[(16384, 11008)] == 1_640_103_936


def test_algorithmic_bytes_rejects(lib):
    assert sq.algorithmic_bytes(-1, 128) == -1
    assert sq.algorithmic_bytes(128, 128, 48) == -1
    assert sq.algorithmic_bytes(128, 128, 256) == -1


@pytest.mark.parametrize("group", [32, 64])
def test_algorithmic_bytes_smaller_groups(lib, group):
    # T = 200, H = 96: 2H/group row groups per token, ceil(200/group) token groups per channel
    T, H = 200, 96
    assert sq.algorithmic_bytes(T, H, group) == 9 * T * H + 4 * T * (2 * H // group) + 4 * H * -(-T // group)


def test_forward_rejects_bad_arguments(lib):
    f = lib.silu_fwd_quant
    assert f(BASE, None, BASE + 2**24, BASE + 2**25, None, 8, 256, 48, None) == 3
    assert f(BASE, None, BASE + 2**24, BASE + 2**25, None, 8, (1 << 22) + 5, 64, None) == 2
    assert f(BASE, None, BASE + 2**24, BASE + 2**25, None, -1, 256, 128, None) == 2
    assert f(BASE, None, BASE + 2**24, BASE + 2**25, None, 2**31 + 1, 8, 128, None) == 2  # past the token limit
    assert f(None, None, BASE + 2**24, BASE + 2**25, None, 8, 256, 128, None) == 1
    assert f(BASE + 8, None, BASE + 2**24, BASE + 2**25, None, 8, 256, 128, None) == 4
    assert f(BASE, BASE + 2**26 + 2, BASE + 2**24, BASE + 2**25, None, 8, 256, 128, None) == 4
    assert f(BASE, None, BASE + 1024, BASE + 2**25, None, 8, 256, 128, None) == 5
    assert f(None, None, None, None, None, 0, 256, 128, None) == 0


def test_forward_q8_1_rejects_bad_arguments(lib):
    f = lib.silu_fwd_quant_q8_1
    assert f(BASE, None, BASE + 2**24, 8, 48, None) == 2      # H not a multiple of 32
    assert f(BASE, None, BASE + 2**24, -1, 64, None) == 2
    assert f(BASE, None, BASE + 2**24, 2**28 + 1, 32, None) == 2  # past the token limit
    assert f(None, None, BASE + 2**24, 8, 64, None) == 1
    assert f(BASE, None, None, 8, 64, None) == 1
    assert f(BASE + 8, None, BASE + 2**24, 8, 64, None) == 4  # x off 16 bytes
    assert f(BASE, None, BASE + 2**24 + 2, 8, 64, None) == 4  # blocks off 4 bytes
    assert f(BASE, BASE + 2**26 + 2, BASE + 2**24, 8, 64, None) == 4
    assert f(BASE, None, BASE + 256, 8, 64, None) == 5        # blocks inside x
    assert f(None, None, None, 0, 64, None) == 0


def test_kquant_swiglu_q8_1_rows_rejects_bad_arguments(lib):
    f = lib.kquant_swiglu_q8_1_rows
    g, u, w, h, q = BASE, BASE + 2**24, BASE + 2**25, BASE + 2**26, BASE + 2**27
    assert f(g, u, None, None, q, 8, 48, None) == 2            # inter not a multiple of 32
    assert f(g, u, None, None, q, -1, 64, None) == 2
    assert f(g, u, None, None, q, 8, (1 << 22) + 32, None) == 2
    assert f(g, u, None, None, q, 2**28 + 1, 32, None) == 2
    assert f(None, u, None, None, q, 8, 64, None) == 1
    assert f(g, None, None, None, q, 8, 64, None) == 1
    assert f(g, u, None, None, None, 8, 64, None) == 1
    assert f(g + 8, u, None, None, q, 8, 64, None) == 4        # gate off 16 bytes
    assert f(g, u + 8, None, None, q, 8, 64, None) == 4
    assert f(g, u, w + 2, None, q, 8, 64, None) == 4
    assert f(g, u, None, h + 8, q, 8, 64, None) == 4
    assert f(g, u, None, None, q + 2, 8, 64, None) == 4
    assert f(g, u, None, None, g + 512, 8, 64, None) == 5      # blocks inside gate
    assert f(g, u, None, u + 64, q, 8, 64, None) == 5          # h inside up
    assert f(g, u, w, h, w + 16, 8, 64, None) == 5             # blocks over the weights
    assert f(g, g, w, h, q, 0, 64, None) == 0                  # nothing to do
    assert f(None, None, None, None, None, 0, 64, None) == 0


def test_gemm_rejects_bad_arguments(lib):
    f = lib.i8_gemm_group_scaled
    A, sA, B, sB, C = BASE, BASE + 2**26, BASE + 2**27, BASE + 2**28, BASE + 2**29
    ok = (A, sA, B, sB, C, 256, 256, 512, 128, 1, 0, None)

    def call(**kw):
        args = list(ok)
        for k, v in kw.items():
            args[["A", "sA", "B", "sB", "C", "M", "N", "K", "group", "bb", "out", "stream"].index(k)] = v
        return f(*args)

    assert call(group=48) == 3 and call(group=256) == 3
    assert call(K=200) == 2 and call(M=-1) == 2 and call(N=-5) == 2 and call(K=-128) == 2
    # K must be a multiple of the group (of 128 only for group 128)
    assert call(K=96, group=64) == 2 and call(K=48, group=32) == 2 and call(K=192) == 2
    assert call(bb=64) == 2 and call(out=2) == 2
    assert call(A=None) == 1 and call(sB=None) == 1 and call(C=None) == 1
    assert call(A=A + 8) == 4 and call(B=B + 4) == 4 and call(sA=sA + 2) == 4 and call(C=C + 2) == 4
    assert call(C=C + 1, out=1) == 4
    assert call(C=A + 64) == 5 and call(C=sB) == 5
    # nothing to do: success without looking at any pointer
    assert call(M=0, A=None, sA=None, B=None, sB=None, C=None) == 0
    assert call(N=0, A=None, sA=None, B=None, sB=None, C=None) == 0


def test_binding_rejects_bad_tensors_before_any_call():
    # shape, rank and device checks raise ValueError on the host, before the
    # library is called (CPU tensors here, so nothing can reach a GPU)
    import torch

    x = torch.zeros((4, 16), dtype=torch.bfloat16)
    dy = torch.zeros((4, 8), dtype=torch.bfloat16)
    outs = sq.empty_outputs(4, 8, "cpu")
    with pytest.raises(ValueError):  # grad_y of rank 1
        sq.silu_dot_fwd_bwd_quant_fuse(x, dy[0], *outs)
    with pytest.raises(ValueError):  # grad_y of rank 0
        sq.silu_dot_fwd_bwd_quant_fuse(x, dy[0, 0], *outs)
    with pytest.raises(ValueError):  # x not [T, 2H]
        sq.silu_dot_fwd_bwd_quant_fuse(x[:, :15], dy, *outs)
    with pytest.raises(ValueError):  # a group the pass does not take
        sq.silu_dot_fwd_bwd_quant_fuse(x, dy, *outs, group_size=16)
    with pytest.raises(ValueError):  # tensors on the host
        sq.silu_dot_fwd_bwd_quant_fuse(x, dy, *outs)
    with pytest.raises(ValueError):  # the bound form checks the same way, once
        sq.bind_backward(x, dy, *outs)
    with pytest.raises(ValueError):
        sq.bind_backward(x[:, :15], dy, *outs)
    with pytest.raises(ValueError):
        sq.silu_fwd_quant(x, outs[0][:, :8], outs[1])
    with pytest.raises(ValueError):
        sq.i8_gemm_group_scaled(outs[0], outs[1], outs[0], outs[1], torch.zeros((4, 4)))
