"""Benchmark of the fused SwiGLU backward + two-axis int8 quantisation pass.

One step = one call of silu_dot_fwd_bwd_quant_fuse over the whole workload
(default: T = 16384 tokens, H = 11008 channels, the largest single-GPU
workload), inputs already resident in HBM.  The metric is achieved HBM
bandwidth: algorithmic bytes per call (reads of x and grad_y, writes of both
code tensors and both scale tensors) divided by the time per call.

Order of a run: inputs drawn on the device; the reference streams (a 1 GiB
copy and a 2-read/1-write bf16 add, for the attainable bandwidth); a settle
phase of about 100 ms running the op on an independent batch of the same
shape, because the device needs some 25-30 ms of this load before its
per-call time stops falling; W warm-up steps on the timed batch; K timed
steps (an event between every two, reported as "steps_us"); 50 more calls for
the per-launch distribution and a cold call; the oracle on the host.

Prints one JSON line.  Usage:
    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--op backward|forward|forward_q8_1|fp8|gemm_dgrad|gemm_wgrad]
                    [--no-cpu-baseline] [--probes before|after|none] [--settle-ms MS]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
KERNEL_SRC = os.path.join(ROOT, "swiglu_backward_int8_amd", "csrc", "siluquant.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


GEMM_SRC = os.path.join(ROOT, "swiglu_backward_int8_amd", "csrc", "i8gemm.hip")


def kernel_source_digest(path: str = KERNEL_SRC) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload: str, src: str = KERNEL_SRC):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("kernel_source_sha") != kernel_source_digest(src):
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_baseline(x, dy, w, min_seconds: float = 10.0, max_calls: int = 5, fp8: bool = False,
                 forward: bool = False, q8_1: bool = False):
    """The oracle, single-threaded, on the whole workload: calls are repeated
    until at least min_seconds of CPU work (at most max_calls); the rate is the
    algorithmic bytes of all calls over their total time (the op's own bytes:
    the backward pass, its E4M3 variant, or the forward quantiser in either
    layout)."""
    import numpy as np
    import torch

    import oracle
    import swiglu_backward_int8_amd as sq

    xb = x.view(torch.int16).cpu().numpy().view(np.uint16)
    db = None if forward else dy.view(torch.int16).cpu().numpy().view(np.uint16)
    oracle.build(force=False)
    calls, total = 0, 0.0
    while calls < max_calls and (calls == 0 or total < min_seconds):
        t = time.perf_counter()
        if forward and q8_1:
            oracle.silu_fwd_quant_q8_1(xb)
        elif forward:
            oracle.silu_fwd_quant(xb)
        else:
            (oracle.silu_dot_fwd_bwd_quant_fuse_fp8 if fp8 else oracle.silu_dot_fwd_bwd_quant_fuse)(xb, db)
        total += time.perf_counter() - t
        calls += 1
    nbytes = (sq.forward_q8_1_bytes(w.T, w.H) if q8_1 else sq.forward_bytes(w.T, w.H)) if forward \
        else sq.algorithmic_bytes(w.T, w.H)
    return {
        "value": round(calls * nbytes / total / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "whole %s workload (T=%d, H=%d), %d call(s), %.1f s single-threaded" % (
            w.name, w.T, w.H, calls, total),
    }


def launch_distribution(step, stream, n: int, dev):
    """After the timed region: per-launch durations of n more calls (an event
    between every two), as median, 10th and 90th percentile, and one cold
    call after 1 GiB of writes has flushed the caches, all in microseconds."""
    import torch

    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    evs[0].record(stream)
    for i in range(n):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    d = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n))
    pick = lambda f: round(d[min(n - 1, int(f * n))], 2)
    flush = torch.empty(2**30, dtype=torch.uint8, device=dev)
    flush.fill_(1)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    step(0)
    c1.record(stream)
    torch.cuda.synchronize()
    del flush
    return {"median": pick(0.5), "p10": pick(0.1), "p90": pick(0.9), "calls": n,
            "cold": round(c0.elapsed_time(c1) * 1e3, 2)}


def host_description() -> dict:
    """The host the CPU baseline ran on: CPU model, logical CPUs, and the CPUs
    this process may use."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def step_series(ms):
    """Per-step durations of the timed region (HIP events between the steps),
    summarised: the first five steps against the rest, and all of them."""
    us = [round(m * 1e3, 1) for m in ms]
    head, tail = us[:5], us[5:]
    return {"first5_mean": round(sum(head) / len(head), 2) if head else None,
            "rest_mean": round(sum(tail) / len(tail), 2) if tail else None,
            "min": min(us) if us else None, "all": us}


def kernel_label(op, H, group=128):
    """The kernel that does the work of one call at channel count H (group
    128): the aligned tiled kernels, or the ones for H not a multiple of the
    group or of 8 (shapes given with --shape)."""
    if op == "forward_q8_1":
        return "silu_fwd_quant_kernel<32, q8_1>"
    if op == "forward":
        if H % 8 and H >= 1024 and 100 * (-(-H // 512) * 512) <= 103 * (-(-H // 128) * 128):
            return "silu_fwd_quant_wide_kernel (rows of 512-channel units, shifted pieces)"
        return "silu_fwd_quant_kernel" + (" (shifted pieces)" if H % 8 else "")
    fmt = "Fmt::kFp8" if op == "fp8" else "Fmt::kInt8"
    if H % 8:
        return "silu_quant_bwd_narrow_kernel<%s>" % fmt
    if H % group:
        return "silu_quant_bwd_%s_kernel<%s>" % ("carry" if H > 128 else "straddle", fmt)
    return "silu_quant_bwd_kernel<%s>" % fmt


def settle(call, ms: float) -> dict:
    """Run the measured op on an independent batch of the same shape (not the
    timed batch) until ms milliseconds have passed.  On MI355X the pass takes
    about 100 calls (25-30 ms) of its own sustained load before its per-call
    time settles (from about 320 us on the first calls to 290 us at
    T = 16384, H = 11008); neither plain copy streams, a bf16 matmul, nor the
    pass at a smaller shape bring the device there, while the pass on another
    batch of the same shape does.  The W warm-up steps then run on the timed
    batch as usual."""
    import torch

    if ms <= 0:
        return {"ms": 0.0, "calls": 0}
    calls = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(10):
            call()
        calls += 10
        torch.cuda.synchronize()
    return {"ms": round((time.perf_counter() - t0) * 1e3, 1), "calls": calls,
            "batch": "an independent batch of the same shape (seed + 500), before the warm-up"}


def stream_probes(dev, reps: int = 50):
    """Plain streaming kernels of known size, for the attainable bandwidth and for
    scaling hardware byte counters: a 1 GiB copy (1 GiB read + 1 GiB written) and
    c = a + b on bf16 (2 reads : 1 write, close to this pass's 1.94 : 1), each
    repeated reps times (about 50 ms of sustained HBM traffic in all)."""
    import torch

    n = 2**30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    a = torch.ones(n // 2, dtype=torch.bfloat16, device=dev)
    b = torch.ones_like(a)
    c = torch.empty_like(a)
    res = {}
    for name, fn, nbytes in (("copy_1GiB", lambda: dst.copy_(src), 2 * n),
                             ("add_bf16_2r1w", lambda: torch.add(a, b, out=c), 3 * n)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / 1e3 / reps
        res[name] = {"bytes": nbytes, "us": round(sec * 1e6, 2), "GB/s": round(nbytes / sec / 1e9, 1)}
    return res


# The two consumers of the pass's outputs at the largest workload (T = 16384,
# H = 11008; D = 4096, the model width that goes with an 11008-wide SwiGLU):
#   dgrad: dX[T, D] = grad_input_q[T, 2H] . Wt[D, 2H]^T, weight scales per 128 x 128 block;
#   wgrad: dW[D, H] = go_q_t[D, T] . y_q_t[H, T]^T, a scale per row of y_q_t and token group.
GEMMS = {
    "gemm_dgrad": dict(M=16384, N=4096, K=22016, b_rows=128, out="bf16"),
    "gemm_wgrad": dict(M=4096, N=11008, K=16384, b_rows=1, out="f32"),
}
PEAK_INT8_TOPS = 5000.0  # MI355X dense int8 matrix peak, published


def gemm_cpu_baseline(A, sA, B, sB, b_rows, min_seconds: float = 10.0):
    """The oracle, single-threaded, on a sample of output rows and columns
    (full K), repeated until at least min_seconds; rate in TOP/s."""
    import numpy as np

    import oracle

    oracle.build(force=False)
    rows, cols = 32, 32
    An, sAn = A[:rows].cpu().numpy(), sA[:rows].cpu().numpy()
    Bn = B[:cols].cpu().numpy()
    sBn = sB.cpu().numpy()[np.arange(cols) // b_rows]
    K = An.shape[1]
    calls, total = 0, 0.0
    while calls == 0 or total < min_seconds:
        t = time.perf_counter()
        oracle.i8_gemm_group_scaled(An, sAn, Bn, sBn)
        total += time.perf_counter() - t
        calls += 1
    return {
        "value": round(calls * 2.0 * rows * cols * K / total / 1e12, 6),
        "unit": "TOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "%d x %d outputs over the full K = %d, %d call(s), %.1f s single-threaded" % (
            rows, cols, K, calls, total),
    }


def run_gemm(args):
    import torch

    import swiglu_backward_int8_amd as sq

    g = GEMMS[args.op]
    M, N, K, b_rows = g["M"], g["N"], g["K"], g["b_rows"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev).manual_seed(7)
    A = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev, generator=gen)
    B = torch.randint(-127, 128, (N, K), dtype=torch.int8, device=dev, generator=gen)
    sA = torch.rand((M, K // 128), device=dev, generator=gen) * 1e-3
    sB = torch.rand((-(-N // b_rows), K // 128), device=dev, generator=gen) * 1e-2
    C = torch.empty((M, N), dtype=torch.bfloat16 if g["out"] == "bf16" else torch.float32, device=dev)

    def step():
        sq.i8_gemm_group_scaled(A, sA, B, sB, C, b_rows_per_scale=b_rows)

    C2 = torch.empty_like(C)
    settle_info = settle(lambda: sq.i8_gemm_group_scaled(A, sA, B, sB, C2, b_rows_per_scale=b_rows), args.settle_ms)
    settle_info["batch"] = "the same operands into a second output, before the warm-up"
    del C2
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_s = ev0.elapsed_time(ev1) / 1e3 / args.steps
    ops = 2.0 * M * N * K
    achieved = ops / per_launch_s / 1e12
    value = ops * args.steps / wall / 1e12
    out = {
        "metric": "achieved int8 TOP/s (+% of MI355X dense int8 peak) for the group-scaled GEMM ("
                  + args.op[5:] + ")",
        "value": round(value, 2),
        "unit": "TOP/s",
        "pct_of_peak": round(100.0 * value / PEAK_INT8_TOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "t16384_h11008_d4096_" + args.op[5:], "M": M, "N": N, "K": K,
                   "b_rows_per_scale": b_rows, "out": g["out"]},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_INT8_TOPS,
            "unit": "TOP/s",
            "frac": round(achieved / PEAK_INT8_TOPS, 4),
            "traffic": measured_traffic(args.op + ":t16384_h11008", GEMM_SRC),
            "kernel": "i8_gemm_kernel",
            "avg_launch_us": round(per_launch_s * 1e6, 3),
        },
        "settle": settle_info,
        "cpu_baseline": None,
    }
    if args.probes != "none":
        out["probes"] = stream_probes(dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = gemm_cpu_baseline(A, sA, B, sB, b_rows)
        out["cpu_baseline"]["host"] = host_description()
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="t16384_h11008")
    ap.add_argument("--shape", default=None, help="T,H of a plain normal workload instead of a named one")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--op", choices=["backward", "forward", "forward_q8_1", "fp8"] + sorted(GEMMS),
                    default="backward",
                    help="backward: the fused SwiGLU backward + two-axis int8 pass (the headline); "
                         "forward: SwiGLU forward + row-wise int8 quantisation; "
                         "forward_q8_1: the same in 32-channel q8_1 blocks; "
                         "fp8: the backward pass with OCP FP8 E4M3 codes; "
                         "gemm_dgrad / gemm_wgrad: the group-scaled int8 GEMMs that consume its outputs")
    ap.add_argument("--graph", choices=["auto", "on", "off"], default="auto",
                    help="replay the K timed steps as one HIP graph (auto: for workloads under 128 MB, whose "
                         "calls take less GPU time than their Python launch)")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="before the warm-up, run the op on an independent batch of the same shape for this "
                         "long, so that the device reaches its steady state under this load (0: skip)")
    ap.add_argument("--probes", choices=["before", "after", "none"], default="before",
                    help="when to time a plain 1 GiB copy and a 2-read/1-write bf16 add (reference streams "
                         "for the attainable bandwidth): before the warm-up (default), after the timed "
                         "region, or not at all")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this pass runs on one GPU; --gpus %d is not supported (the tensors of a "
              "multi-GPU job shard by tokens with no exchange, so per-GPU throughput is the "
              "one-GPU figure)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    if args.op in GEMMS:
        return run_gemm(args)

    import torch

    import swiglu_backward_int8_amd as sq
    from swiglu_backward_int8_amd.inputs import WORKLOADS, Workload, make_inputs

    w = WORKLOADS[args.workload]
    if args.shape:
        # a plain normal workload of another shape (channel shards, ragged H), for profiling
        T_, H_ = (int(v) for v in args.shape.split(","))
        w = Workload("t%d_h%d" % (T_, H_), T_, H_, ("normal", 1.0), ("normal", 1.0), ("normal", 0.01), seed=11)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q8_1 = args.op == "forward_q8_1"
    forward = args.op == "forward" or q8_1
    fp8 = args.op == "fp8"
    nbytes = (sq.forward_q8_1_bytes(w.T, w.H) if q8_1 else sq.forward_bytes(w.T, w.H)) if forward \
        else sq.algorithmic_bytes(w.T, w.H)
    # Rotate buffer sets so that one pass over them exceeds twice the 256 MB
    # last-level cache: every step then reads its inputs from HBM.
    sets = max(1, -(-512 * 2**20 // nbytes))
    # The timed batch is the workload's own draw; the other sets are row blocks
    # of one tall draw with the same distributions (a few kernels instead of a
    # draw per set, which matters under a counter profiler), each starting on
    # 16 bytes; one more, independent batch of the same shape for the settle
    # phase.
    batches = [make_inputs(w, device=dev, seed=w.seed)]
    if sets > 1:
        t_pad = -(-w.T // 8) * 8
        xa, dya = make_inputs(w, device=dev, seed=w.seed + 1000, T=(sets - 1) * t_pad)
        batches += [(xa[r * t_pad:r * t_pad + w.T], dya[r * t_pad:r * t_pad + w.T]) for r in range(sets - 1)]
    batches.append(make_inputs(w, device=dev, seed=w.seed + 500 * 1000))
    if forward:
        batches = [(x, None) for x, _ in batches]
    bufs = []
    for x, dy in batches:
        if q8_1:
            bufs.append((x, None, (torch.empty((w.T, (w.H // 32) * sq.Q8_1_BLOCK), dtype=torch.uint8, device=dev),)))
        elif forward:
            outs = (torch.empty((w.T, w.H), dtype=torch.int8, device=dev),
                    torch.empty((w.T, -(-w.H // 128)), dtype=torch.float32, device=dev))
            bufs.append((x, None, outs))
        else:
            bufs.append((x, dy, sq.empty_outputs(w.T, w.H, dev, fp8=fp8)))
    settle_batch = bufs.pop()
    sq.prepare()
    torch.cuda.synchronize()
    # The pass and its E4M3 variant go through calls bound once per buffer set:
    # the binding checks the tensors when binding, not on every call, so the
    # first timed step does not carry the checks' host time while the device
    # waits for it.
    bound = {}
    if not (q8_1 or forward):
        for k, (x, dy, outs) in enumerate(bufs + [settle_batch]):
            bound[k] = sq.bind_backward(x, dy, *outs, fp8=fp8)

    def step(i, batch=None):
        k = len(bufs) if batch is not None else i % sets
        x, dy, outs = batch if batch is not None else bufs[k]
        if q8_1:
            sq.silu_fwd_quant_q8_1(x, *outs)
        elif forward:
            sq.silu_fwd_quant(x, *outs)
        else:
            bound[k]()

    probes = None
    if args.probes == "before":
        probes = stream_probes(dev)
    settle_info = settle(lambda: step(0, settle_batch), args.settle_ms)
    use_graph = args.graph == "on" or (args.graph == "auto" and nbytes < 128 * 2**20)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)  # the stream every call is launched on
    if use_graph:
        # Small workloads: a call takes less GPU time than the Python binding
        # takes to launch it, so the K steps are captured in one HIP graph and
        # replayed (once untimed, then once timed); the GPU time is then the
        # kernels' and not the host's.  Per-step times are not taken.
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for i in range(args.steps):
                    step(i)
        stream.wait_stream(side)
        g.replay()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu_ms = ev0.elapsed_time(ev1)
        series = {"graph": True, "note": "K steps replayed as one HIP graph; no per-step events"}
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        evs[0].record(stream)
        for i in range(args.steps):
            step(i)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu_ms = evs[0].elapsed_time(evs[-1])
        series = step_series([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])

    per_launch_s = gpu_ms / 1e3 / args.steps
    achieved = nbytes / per_launch_s / 1e9
    value = nbytes * args.steps / wall / 1e9
    timing = launch_distribution(step, stream, min(args.steps, 50), dev)
    metric = "achieved HBM GB/s (+% of MI355X peak) for fused silu fwd/bwd+int8 quant"
    if q8_1:
        metric = "achieved HBM GB/s (+% of MI355X peak) for fused silu forward + q8_1 block quant"
    elif forward:
        metric = "achieved HBM GB/s (+% of MI355X peak) for fused silu forward + row-wise int8 quant"
    elif fp8:
        metric = "achieved HBM GB/s (+% of MI355X peak) for fused silu fwd/bwd+fp8 e4m3 quant"
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "GB/s",
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "T": w.T, "H": w.H, "group": 32 if q8_1 else 128,
            "bytes_per_step": nbytes, "pairs_per_s": round(w.T * w.H * args.steps / wall, 1),
            "input_elements_per_s": round((2 if args.op.startswith("forward") else 3) * w.T * w.H * args.steps / wall, 1),
            "buffer_sets": sets,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic({"forward": "forward:", "forward_q8_1": "forward_q8_1:", "fp8": "fp8:"}.get(
                args.op, "") + w.name),
            "kernel": kernel_label(args.op, w.H),
            "avg_launch_us": round(per_launch_s * 1e6, 3),
        },
        "settle": settle_info,
        "steps_us": series,
        "launch_us": timing,
        "cpu_baseline": None,
    }
    if args.probes == "after":
        probes = stream_probes(dev)
    if probes is not None:
        out["probes"] = probes
    if not args.no_cpu_baseline:
        x, dy, _ = bufs[0]
        out["cpu_baseline"] = cpu_baseline(x, dy, w, fp8=fp8, forward=forward, q8_1=q8_1)
        out["cpu_baseline"]["host"] = host_description()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
