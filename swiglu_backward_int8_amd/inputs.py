"""Seeded synthetic inputs for the fused SwiGLU backward + int8 quantisation pass.

This module draws random numbers and rounds them to bf16; it holds none of the
pass's own arithmetic, so the same inputs can feed both the HIP path and the
CPU oracle.  Generation runs on whatever device the caller names (``cuda`` for
the large workloads, ``cpu`` for small ones); each tensor has its own seeded
``torch.Generator`` so that a tensor does not depend on the order the others
were drawn in.  The same seed on the same device type gives the same bits.

Workloads (normal parameters are (mean, standard deviation)):

=========================  ======  ======  ===================  ==================  ===========  ==========================
name                       T       H       gate                 up                  grad_y       structure
=========================  ======  ======  ===================  ==================  ===========  ==========================
t256_h256                  256     256     N(0, 1)              N(0, 1)             N(0, 0.01)   --
t4096_h1408                4096    1408    N(0, 1)              N(0, 1)             N(0, 0.01)   --
t8192_h4096                8192    4096    N(0, 2)              N(0, 1)             N(0, 1e-3)   --
t16384_h11008              16384   11008   N(0, 1)              N(0, 1)             N(0, 0.01)   --
t32768_h2048_outliers      32768   2048    Student-t(3)         Student-t(3)        N(0, 0.01)   0.1% of gate/up x100,
                                                                                                  rows t % 97 == 96 zero
=========================  ======  ======  ===================  ==================  ===========  ==========================

Student-t with 3 degrees of freedom is drawn as z0 / sqrt((z1^2 + z2^2 + z3^2) / 3)
from four independent standard normals.  The outlier mask is an independent
Bernoulli(0.001) per element of gate and of up, applied before the bf16
rounding.  Zeroed rows are zero in both x and grad_y.
"""

from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    gate: tuple  # ("normal", std) or ("student_t3", scale)
    up: tuple
    grad_y: tuple
    seed: int
    outlier_p: float = 0.0
    outlier_mult: float = 1.0
    zero_row_period: int = 0  # rows t with t % period == period - 1 are zero

    @property
    def pairs(self) -> int:
        return self.T * self.H


WORKLOADS = {
    w.name: w
    for w in [
        Workload("t256_h256", 256, 256, ("normal", 1.0), ("normal", 1.0), ("normal", 0.01), seed=0),
        Workload("t4096_h1408", 4096, 1408, ("normal", 1.0), ("normal", 1.0), ("normal", 0.01), seed=1),
        Workload("t8192_h4096", 8192, 4096, ("normal", 2.0), ("normal", 1.0), ("normal", 1e-3), seed=2),
        Workload("t16384_h11008", 16384, 11008, ("normal", 1.0), ("normal", 1.0), ("normal", 0.01), seed=3),
        Workload("t32768_h2048_outliers", 32768, 2048, ("student_t3", 1.0), ("student_t3", 1.0),
                 ("normal", 0.01), seed=4, outlier_p=1e-3, outlier_mult=100.0, zero_row_period=97),
    ]
}

# Streams of random numbers, one per tensor.
_GATE, _UP, _DY, _GATE_MASK, _UP_MASK = range(5)


def _gen(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 64 + stream)
    return g


def _draw(kind: tuple, shape, device, gen: torch.Generator) -> torch.Tensor:
    dist, param = kind
    if dist == "normal":
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * param
    if dist == "student_t3":
        z = torch.randn((4,) + tuple(shape), generator=gen, device=device, dtype=torch.float32)
        chi2 = z[1] * z[1] + z[2] * z[2] + z[3] * z[3]
        return z[0] / torch.sqrt(chi2 / 3.0) * param
    raise ValueError("unknown distribution %r" % (dist,))


def make_inputs(w: Workload | str, device="cpu", seed: int | None = None, T: int | None = None):
    """Return (x [T, 2H] bf16, grad_y [T, H] bf16) for a workload on ``device``.

    ``seed`` overrides the workload's own seed (a second-seed run); ``T``
    overrides the token count (a cut-down copy with the same distributions).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    seed = w.seed if seed is None else seed
    T = w.T if T is None else T
    H = w.H
    x = torch.empty((T, 2 * H), dtype=torch.bfloat16, device=device)
    for half, kind, stream, mstream in ((0, w.gate, _GATE, _GATE_MASK), (1, w.up, _UP, _UP_MASK)):
        v = _draw(kind, (T, H), device, _gen(device, seed, stream))
        if w.outlier_p > 0.0:
            m = torch.rand((T, H), generator=_gen(device, seed, mstream), device=device) < w.outlier_p
            v = torch.where(m, v * w.outlier_mult, v)
        x[:, half * H:(half + 1) * H] = v.to(torch.bfloat16)
        del v
    grad_y = _draw(w.grad_y, (T, H), device, _gen(device, seed, _DY)).to(torch.bfloat16)
    if w.zero_row_period > 0:
        rows = torch.arange(T, device=device) % w.zero_row_period == w.zero_row_period - 1
        x[rows] = 0
        grad_y[rows] = 0
    return x, grad_y


def random_inputs(T: int, H: int, device="cpu", seed: int = 0, gate_std: float = 1.0,
                  up_std: float = 1.0, dy_std: float = 0.01):
    """Plain normal inputs of any shape (for parity cases beyond the named workloads)."""
    w = Workload("custom", T, H, ("normal", gate_std), ("normal", up_std), ("normal", dy_std), seed=seed)
    return make_inputs(w, device=device)
