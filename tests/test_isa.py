"""Checks of the gfx950 instructions our own build generates (CPU only: hipcc
compiles the sources to assembly with the library's flags; nothing runs).

* No packed fp32 arithmetic (v_pk_fma_f32, v_pk_mul_f32, v_pk_add_f32) in
  any kernel: the build turns the feature off, and the values must come from
  scalar fp32 operations in the written order.
* In the fused pass and the forward quantisers every fused multiply-add
  (v_fma_f32, v_fmac_f32, v_fmamk/fmaak_f32, v_fma_mix*) belongs either to an
  IEEE division sequence (v_div_scale_f32 ... v_div_fixup_f32, the scale and
  inverse of a group whose maximum is below 2^-119) or to the compiler's
  expansion of a 64-bit integer division in the index arithmetic (it scales by
  2^32, the literal 0x4f800000 or 0xcf800000): the elementwise formulas, the
  bf16 round trips, the code rounding and the q8_1 sums are separate
  multiplies, adds and conversions, which is what the oracle computes
  (evaluation order of d_gate, rounding of the fp32 product v * inv, fl32 of
  a block's scale times its code sum before binary16).  "Belongs to a
  division sequence" is checked as: within 20 instructions of a division
  instruction.  The GEMM is exempt: its promotion is a stated fma.
* The aligned pass, the forward quantisers and the GEMM spill no registers
  and use no scratch memory.  (The straddling-group carry kernel is known to
  spill 2-8 registers at some group sizes and is not held to this.)
"""

import os
import re
import shutil

import pytest

from swiglu_backward_int8_amd import _build

pytestmark = pytest.mark.skipif(not os.path.exists(_build.hipcc()) and shutil.which("hipcc") is None,
                                reason="hipcc is not installed")

SRC = {name: os.path.join(_build.PKG, "csrc", name) for name in ("siluquant.hip", "i8gemm.hip")}
PACKED = re.compile(r"\bv_pk_(fma|mul|add)_f32\b")
FMA = re.compile(r"\bv_(fma_f32|fmac_f32|fmamk_f32|fmaak_f32|fma_mix\w*|mad_f32|mac_f32|madmk_f32|madak_f32|mad_mix\w*)\b")
INT_DIV = re.compile(r"0x[4c]f800000\b")  # 2^32 scaling in the compiler's 64-bit integer division
DIV = re.compile(r"\bv_div_(scale|fmas|fixup)_f32\b")


def kernels(asm: str) -> dict:
    """kernel symbol -> its instruction lines (label to s_endpgm)."""
    out, name = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            name = m.group(1)
            out[name] = []
            continue
        if name is None:
            continue
        s = line.strip()
        if s and not s.startswith((";", ".", "//")) and not s.endswith(":"):
            out[name].append(s)
        if s.startswith("s_endpgm"):
            name = None
    return {k: v for k, v in out.items() if v}


def metadata(asm: str) -> dict:
    """kernel symbol -> (private segment bytes, VGPR spills, SGPR spills)."""
    meta = {}
    for m in re.finditer(r"\.name:\s+(\S+)(.*?)(?=\n\s+- \.|\n\s*\.end_amdgpu_metadata)", asm, re.S):
        body = m.group(2)
        get = lambda key: int(re.search(r"\." + key + r":\s+(\d+)", body).group(1))
        meta[m.group(1)] = (get("private_segment_fixed_size"), get("vgpr_spill_count"), get("sgpr_spill_count"))
    return meta


@pytest.fixture(scope="module")
def asm():
    return {name: _build.device_asm(path) for name, path in SRC.items()}


def test_every_kernel_is_found(asm):
    k = kernels(asm["siluquant.hip"])
    assert any("silu_quant_bwd_kernel" in n for n in k)
    assert any("silu_fwd_quant_kernel" in n for n in k)
    assert sum("i8_gemm_kernel" in n for n in kernels(asm["i8gemm.hip"])) == 12


def test_no_packed_fp32_arithmetic(asm):
    for src, text in asm.items():
        for name, body in kernels(text).items():
            bad = [l for l in body if PACKED.search(l)]
            assert not bad, "%s: %s in %s" % (src, bad[:3], name)


def test_pass_and_forward_fmas_only_in_divisions(asm):
    checked = 0
    for name, body in kernels(asm["siluquant.hip"]).items():
        if "silu_quant_bwd" not in name and "silu_fwd_quant" not in name:
            continue
        divs = [i for i, l in enumerate(body) if DIV.search(l)]
        for i, l in enumerate(body):
            if FMA.search(l) and not INT_DIV.search(l):
                assert any(abs(i - d) <= 20 for d in divs), "%s: '%s' outside a division" % (name, l)
                checked += 1
    assert checked > 0  # the division fallbacks exist and were seen


def test_pass_and_forward_use_no_fused_conversions(asm):
    # conversions that multiply by a scale, or dot products of fp values,
    # would round a product once where the oracle rounds it to fp32 first
    fused = re.compile(r"\bv_(cvt_scalef32\w*|dot2\w*_f32\w*|dot2c_f32\w*)\b")
    for name, body in kernels(asm["siluquant.hip"]).items():
        bad = [l for l in body if fused.search(l)]
        assert not bad, "%s: %s" % (name, bad[:3])


def test_hot_kernels_do_not_spill(asm):
    meta = {**metadata(asm["siluquant.hip"]), **metadata(asm["i8gemm.hip"])}
    hot = [n for n in meta if re.search(r"silu_quant_bwd_kernel|silu_fwd_quant_kernel|silu_fwd_quant_wide_kernel|"
                                        r"i8_gemm_kernel", n)]
    assert len(hot) >= 12 + 6
    for name in hot:
        private, vgpr_spill, _ = meta[name]
        assert private == 0 and vgpr_spill == 0, "%s: %d bytes of scratch, %d VGPR spills" % (name, private,
                                                                                            vgpr_spill)
