"""Benchmark of the dense decode GEMV on MI355X: IQ4_NL 8192 x 2560 weights x q8_1 activations at
1, 4 and 8 columns, on cold weights.

One step = the hot path once per column count n in (1, 4, 8): q8_1 quantization of the n
activation columns, then the n-column GEMV over the next weight copy of a rotation.  The
rotation holds enough copies (44 x 11.8 MB = 519 MB) to exceed twice the 256 MB Infinity Cache,
so every GEMV reads its weights from HBM.  The six launches of a step are replayed from a HIP
graph (one graph per rotation slot); inputs are resident in HBM before the timed region.

Prints one JSON line (see the fields below).  `value` is the step's algorithmic bytes (weights,
q8_1 activations, fp32 outputs, quantizer reads/writes) divided by the step time.  `roofline` is
the GEMV kernel's algorithmic bytes per launch over its average launch duration, timed with HIP
events on the launch stream around graph-batched launches of each column count.
`cpu_baseline` times the CPU oracle on the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-graph] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
NROWS, K = 8192, 2560
COLS = (1, 4, 8)
NCOPIES = 44            # 44 x 11,796,480 B = 519 MB > 2 x 256 MB Infinity Cache
NDISTINCT = 6           # distinct seeded copies; the rest of the rotation repeats them at other addresses


def gemv_bytes(n: int) -> int:
    """Algorithmic bytes of one n-column GEMV: every weight byte once, n q8_1 columns, n fp32 rows."""
    return NROWS * (K // 32) * 18 + n * (K // 32) * 36 + n * NROWS * 4


def quant_bytes(n: int) -> int:
    return n * K * 4 + n * (K // 32) * 36


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--batch-reps", type=int, default=5, help="graph replays per column count for the roofline timing")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the decode GEMV is measured on one "
              "GPU's share; see the design notes for how it would shard.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import moe_expert_amd as M
    import synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    t0 = time.time()
    host_copies = [synth.iq4nl_weights(synth.rng_for(synth.SEEDS["iq4nl_8192x2560"] + i), NROWS, K)
                   for i in range(NDISTINCT)]
    copies = [torch.from_numpy(host_copies[i % NDISTINCT]).to(dev) for i in range(NCOPIES)]
    rng = synth.rng_for(synth.SEEDS["iq4nl_8192x2560"] + 100)
    xs = {n: torch.from_numpy(synth.activations(rng, n, K)).to(dev) for n in COLS}
    xqs = {n: torch.empty((n, (K // 32) * 36), dtype=torch.uint8, device=dev) for n in COLS}
    ys = {n: torch.empty((n, NROWS), dtype=torch.float32, device=dev) for n in COLS}
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    def step(slot: int):
        w = copies[slot % NCOPIES]
        for n in COLS:
            M.qmm_quantize_q8_1(xs[n], out=xqs[n])
            M.qgemv_dense(M.QMM_IQ4_NL, w, NROWS, K, xqs[n], n, y=ys[n])

    def gemv_batch(n: int):
        for i in range(NCOPIES):
            M.qgemv_dense(M.QMM_IQ4_NL, copies[i], NROWS, K, xqs[n], n, y=ys[n])

    use_graph = not args.no_graph
    side = torch.cuda.Stream()
    graphs, batch_graphs = [], {}
    if use_graph:
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0)
            for n in COLS:
                gemv_batch(n)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for slot in range(NCOPIES):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(slot)
            graphs.append(g)
        for n in COLS:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                gemv_batch(n)
            batch_graphs[n] = g
        torch.cuda.synchronize()

    def run_step(i: int):
        if use_graph:
            graphs[i % NCOPIES].replay()
        else:
            step(i)

    # ---- the contract: W untimed steps, then exactly K timed steps between synchronisations
    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        run_step(args.warmup + i)
    stop.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(stop) / args.steps
    step_bytes = sum(gemv_bytes(n) + quant_bytes(n) for n in COLS)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # ---- GEMV launches alone, graph-batched over the cold rotation, HIP events on the launch stream
    us_per_call, gbps = {}, {}
    tot_bytes = tot_us = 0.0
    for n in COLS:
        run = (batch_graphs[n].replay if use_graph else (lambda n=n: gemv_batch(n)))
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.batch_reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (args.batch_reps * NCOPIES)
        us_per_call[str(n)] = round(us, 3)
        gbps[str(n)] = round(gemv_bytes(n) / (us * 1e-6) / 1e9, 1)
        tot_bytes += gemv_bytes(n)
        tot_us += us
    achieved = tot_bytes / (tot_us * 1e-6) / 1e9

    # ---- warm context: one copy, repeated (largely served from the Infinity Cache), graph-batched
    warm = {}
    for n in COLS:
        def warm_batch(n=n):
            for _ in range(NCOPIES):
                M.qgemv_dense(M.QMM_IQ4_NL, copies[0], NROWS, K, xqs[n], n, y=ys[n])
        if use_graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                warm_batch()
            run = g.replay
        else:
            run = warm_batch
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.batch_reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        warm[str(n)] = round(e0.elapsed_time(e1) * 1e3 / (args.batch_reps * NCOPIES), 3)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(host_copies[0], step_bytes)

    out = {
        "metric": "µs/call and achieved HBM GB/s, IQ4_NL 8192x2560 GEMV at 1/4/8 columns",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "IQ4_NL dense decode GEMV 8192x2560 x q8_1, 1/4/8 columns, cold rotation of "
                               f"{NCOPIES} weight copies ({NCOPIES * NROWS * (K // 32) * 18 / 1e6:.0f} MB)",
                   "nrows": NROWS, "k": K, "columns": list(COLS), "weight_copies": NCOPIES,
                   "hip_graph": use_graph},
        "us_per_call": us_per_call,
        "gbps_per_call": gbps,
        "warm_us_per_call": warm,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "gemv_kernel<IQ4_NL> (1, 4, 8 columns)"},
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline(w_host, step_bytes: int, min_s: float = 10.0) -> dict:
    """The oracle on the same step (all 8192 rows at 1, 4 and 8 columns, plus the quantizer),
    repeated until about ``min_s`` seconds of CPU work have run."""
    import oracle
    import synth
    rng = synth.rng_for(synth.SEEDS["iq4nl_8192x2560"] + 100)
    xs = {n: synth.activations(rng, n, K) for n in COLS}
    reps = 0
    t0 = time.perf_counter()
    while True:
        for n in COLS:
            xq = oracle.quantize_q8_1(xs[n])
            oracle.gemv(oracle.IQ4_NL, w_host, K, xq)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_s:
            break
    per_step = dt / reps
    return {"value": round(step_bytes / per_step / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"the full step (8192 rows at 1/4/8 columns + q8_1 of the columns) x {reps} repetitions, "
                      f"{dt:.1f} s, {per_step * 1e3:.1f} ms per step"}


if __name__ == "__main__":
    sys.exit(main())
