"""The first call of a process, captured into a HIP graph (GPU).

The library keeps no state and never waits: its sigmoid table is constant data
of the code object, and every call only checks its arguments, asks for the
device's compute-unit count and enqueues kernels on the caller's stream.  So
even the very first call a process makes can be captured.  A fresh child
process captures the pass as its first call into the library, replays the
graph on two inputs (with eager work between the replays) and saves the
outputs; this process checks each replay against the oracle.
"""

import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest

import oracle
from swiglu_backward_int8_amd.inputs import random_inputs

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
T, H = 512, 1408
SEEDS = (61, 62)

CHILD = textwrap.dedent("""
    import sys
    import numpy as np
    import torch
    sys.path.insert(0, %(root)r)
    import swiglu_backward_int8_amd as sq
    from swiglu_backward_int8_amd.inputs import random_inputs

    dev = "cuda:0"
    T, H = %(T)d, %(H)d
    x = torch.empty((T, 2 * H), dtype=torch.bfloat16, device=dev)
    dy = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    outs = sq.empty_outputs(T, H, dev)
    torch.cuda.synchronize()
    print("capturing the first call", flush=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sq.silu_dot_fwd_bwd_quant_fuse(x, dy, *outs)
    saved = {}
    for seed in %(seeds)r:
        x2, dy2 = random_inputs(T, H, device=dev, seed=seed)
        x.copy_(x2)
        dy.copy_(dy2)
        for o in outs:
            o.fill_(-7 if o.dtype == torch.int8 else float("nan"))
        g.replay()
        torch.cuda.synchronize()
        print("replayed seed", seed, flush=True)
        for name, o in zip(("gq", "gs", "yq", "ys"), outs):
            saved["%%s_%%d" %% (name, seed)] = o.cpu().numpy()
    np.savez(sys.argv[1], **saved)
    print("done", flush=True)
""")


def test_first_call_captured_in_a_graph(tmp_path):
    script = tmp_path / "first_call.py"
    script.write_text(CHILD % {"root": ROOT, "T": T, "H": H, "seeds": SEEDS})
    out = tmp_path / "outs.npz"
    r = subprocess.run([sys.executable, str(script), str(out)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    got = np.load(out)
    for seed in SEEDS:
        x, dy = random_inputs(T, H, device="cuda:0", seed=seed)
        bits = lambda t: t.contiguous().view(__import__("torch").int16).cpu().numpy().view(np.uint16)
        want = oracle.silu_dot_fwd_bwd_quant_fuse(bits(x), bits(dy))
        for name, w in zip(("gq", "gs", "yq", "ys"), want):
            g = got["%s_%d" % (name, seed)]
            assert g.shape == w.shape
            assert np.array_equal(g, w), "%s differs from the oracle on replay of seed %d" % (name, seed)
