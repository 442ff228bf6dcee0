"""Build step for libsiluquant.so (in-tree, for gfx950).

sigmoid_table.py writes the kernels' sigmoid table into _build/, then hipcc
compiles the HIP sources (the fused SwiGLU passes and the group-scaled int8
GEMM) into one shared library next to this file.
Flags that matter for the numbers the library produces:
  -ffp-contract=off                  no fused multiply-add: the arithmetic order
                                     is the one written in the source;
  -fno-gpu-flush-denormals-to-zero   fp32 subnormals are kept;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                     no packed fp32 instructions.
"""

from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
GEN = os.path.join(PKG, "_build")  # generated sources (not tracked)
SRCS = [os.path.join(PKG, "csrc", "siluquant.hip"), os.path.join(PKG, "csrc", "i8gemm.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsiluquant.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False) -> str:
    """Generate the sigmoid table, compile libsiluquant.so for gfx950 and
    return its path."""
    from swiglu_backward_int8_amd import sigmoid_table

    sigmoid_table.write(os.path.join(GEN, "sigmoid_table.inc"))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I" + INCLUDE, "-I" + GEN] + SRCS + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (r.returncode, err))
    if verbose and err.strip():
        print(err)
    os.replace(tmp, LIB)
    return LIB


def device_asm(src: str) -> str:
    """gfx950 assembly of one HIP source, compiled with the library's flags
    (for checks of the generated instructions)."""
    from swiglu_backward_int8_amd import sigmoid_table
    import tempfile

    sigmoid_table.write(os.path.join(GEN, "sigmoid_table.inc"))
    flags = [f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [hipcc()] + flags + ["--cuda-device-only", "-S", "-I" + INCLUDE, "-I" + GEN, src, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc -S failed (%d):\n%s" % (r.returncode, r.stderr))
        with open(out) as f:
            return f.read()


if __name__ == "__main__":
    print(build(verbose=True))
