"""How often three readings of the quantiser's rounding step give different
int8 codes on the synthetic workloads -- TEST INFRASTRUCTURE ONLY.

The page "kernelgen-challenge-9-task3-silu-quant" (githubhelp.com, its list of
design constraints) asks the quantiser to multiply by a precomputed inverse
scale.  With the bf16 value v, scale = amax / 127 and inv = 1 / scale (both
fp32), the code is the nearest integer (ties to even) of one of:

    fp32   the fp32 product RN(v * inv)          (the oracle's reading)
    exact  the exact product v * inv             (an FMA with a rounding offset)
    div    the fp32 quotient RN(v / scale)       (no inverse at all)

This script takes the oracle's own bf16 intermediates and scales, forms the
codes under each reading with numpy, and prints, per workload and output
tensor, the fraction of codes in which each pair of readings differs (the
difference is always one step).  Inputs are generated on the CPU with the
workloads' distributions and seeds; the two largest workloads are processed
in slices of 1024 tokens so that memory stays bounded.

    python tests/rule_rates.py [workload ...]
"""

from __future__ import annotations

import os
import sys

import numpy as np

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

import oracle  # noqa: E402  (the checker; this script is test tooling)

READINGS = ("fp32", "exact", "div")


def _codes(v: np.ndarray, scale: np.ndarray, reading: str) -> np.ndarray:
    """Codes of bf16-valued v (float32) for broadcastable fp32 scales."""
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        inv = (np.float32(1.0) / scale).astype(np.float32)
        if reading == "fp32":
            p = (v * inv).astype(np.float32)
        elif reading == "exact":
            # 8 significant bits times 24: exact in double
            p = v.astype(np.float64) * inv.astype(np.float64)
        else:
            p = (v / scale).astype(np.float32)
        q = np.clip(np.rint(p), -127.0, 127.0)
    q[v == 0.0] = 0.0
    return q.astype(np.int8)


def _compare(v: np.ndarray, scale: np.ndarray, counts: dict) -> None:
    q = {r: _codes(v, scale, r) for r in READINGS}
    for a in range(len(READINGS)):
        for b in range(a + 1, len(READINGS)):
            d = np.abs(q[READINGS[a]].astype(np.int16) - q[READINGS[b]].astype(np.int16))
            key = READINGS[a] + "/" + READINGS[b]
            counts[key] = counts.get(key, 0) + int(np.count_nonzero(d))
            counts["maxdiff"] = max(counts.get("maxdiff", 0), int(d.max()) if d.size else 0)
    counts["n"] = counts.get("n", 0) + v.size


def rates(name: str, chunk: int = 1024) -> dict:
    from swiglu_backward_int8_amd.inputs import WORKLOADS, make_inputs

    w = WORKLOADS[name]
    x, dy = make_inputs(w, device="cpu")
    G = oracle.GROUP
    rows, cols = {}, {}
    for t0 in range(0, w.T, chunk):
        xs, ds = x[t0:t0 + chunk], dy[t0:t0 + chunk]
        Y, D = oracle.intermediates(xs, ds)
        _, gs, _, ys = oracle.quantise(Y, D)
        T = Y.shape[0]
        # row groups: G consecutive positions of the 2H-long row
        _compare(D.reshape(T, -1, G), gs[:, :, None], rows)
        # token groups of y^T: G consecutive tokens of one channel
        _compare(Y.reshape(T // G, G, -1), ys.T[:, None, :], cols)
    return {"grad_input_q": rows, "y_q_t": cols}


def main(names) -> None:
    for name in names:
        r = rates(name)
        for tensor, c in r.items():
            n = c["n"]
            print("%-24s %-12s codes %12d  " % (name, tensor, n)
                  + "  ".join("%s %.3e" % (k, c[k] / n) for k in c if "/" in k)
                  + "  max |dq| %d" % c["maxdiff"], flush=True)


if __name__ == "__main__":
    from swiglu_backward_int8_amd.inputs import WORKLOADS

    main(sys.argv[1:] or list(WORKLOADS))
