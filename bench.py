"""Benchmark of the block-quantized hot path on one MI355X.

Headline workload: dense decode GEMV, IQ4_NL 8192 x 2560 weights at 1, 4 and 8 activation
columns, on cold weights.  One step = the hot path once per column count n in (1, 4, 8): the
one-column call takes its fp32 column and forms q8_1 inside the GEMV (one launch); the 4- and
8-column calls quantize their columns to q8_1 and run the q8_1 GEMV.  Each step reads the next
weight copy of a rotation whose total (47 copies, 554 MB) exceeds twice the 256 MB Infinity
Cache, so every GEMV reads its weights from HBM.  The launches of a step are replayed from a HIP
graph (one per rotation slot, each replayed once before timing); inputs are resident in HBM
before the timed region.

The default run (--workload all) prints ONE JSON line: the headline fields, and under
"configs" every other workload timed the same way: Q8_0 512 x 2560 at 1 column, Q8_0
12288 x 2560 at 1-4 columns, Q8_0 2560 x 6144 at 7-8 columns, the grouped MoE decode (128
experts, 16 groups x m entries, m = 1/4/8) and the prefill grouped expert GEMM (8192 tokens x
2560, top-8 of 128 experts).  --workload gemv|tiny|q8_0|grouped|prefill runs one of them alone.

Fields: `value` = algorithmic bytes (GEMV, grouped) or FLOPs (prefill) of a step / step time;
`roofline` = algorithmic bytes or FLOPs per launch of the kernels the step runs over their
average launch duration, timed with HIP events on the launch stream around graph-batched
launches of the cold rotation; `cpu_baseline` = the CPU oracle on the same workload (or a stated
sample of it), on all host threads and on one.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload W] [--no-graph] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2516.6
MALL_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
CALIB_BYTES = 64 << 20   # the plain copy that scales the counters


# Library sources each workload's kernels are built from: a recorded counter figure is reported
# only while these hash as they did when the counters were taken.
DIGEST_SOURCES = {
    "gemv": ("qmm_host.h", "qmm_device.h", "qmm_gemv.h", "qmm_gemv.hip"),
    "grouped": ("qmm_host.h", "qmm_device.h", "qmm_gemv.h", "qmm_grouped.hip"),
    "prefill": ("qmm_host.h", "qmm_device.h", "qmm_gemv.h", "qmm_prefill.hip"),
    "combine": ("qmm_host.h", "qmm_device.h", "qmm_combine.hip"),
}
DIGEST_SOURCES["q8_0"] = DIGEST_SOURCES["planes"] = DIGEST_SOURCES["gemv"]
DIGEST_SOURCES["dense"] = DIGEST_SOURCES["mmq"] = DIGEST_SOURCES["prefill"]


def source_digest(files=None):
    """sha256 of the library sources `files` (names under moe_expert_amd/csrc; default: all of
    them and the header)."""
    import hashlib
    h = hashlib.sha256()
    if files is None:
        paths = [os.path.join(d, f) for d in ("moe_expert_amd/csrc", "include")
                 for f in sorted(os.listdir(os.path.join(ROOT, d)))]
    else:
        paths = [os.path.join("moe_expert_amd/csrc", f) for f in files]
    for rel in paths:
        h.update(os.path.basename(rel).encode())
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(key):
    """HBM bytes per launch recorded for `key` by --pmc-summary, or None when there is no record
    or the sources it was taken on have changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_digest(rec.get("sources")):
        return None
    return rec


def timed_graph(torch, fn, reps, use_graph=True):
    """Average ms of fn() over `reps` runs after one warm run; graph-captured when use_graph."""
    if use_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        run = g.replay
    else:
        run = fn
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def contract_steps(torch, run_step, steps, warmup):
    """W untimed steps, then exactly K timed steps between synchronisations; ms per step."""
    for i in range(warmup):
        run_step(i)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        run_step(warmup + i)
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def capture_slots(torch, step, nslots):
    """One HIP graph per rotation slot of `step`, each replayed once here (its first replay
    uploads it: set-up, not timed work); returns run_step(i).  The replays go in rotation order,
    so the slots the timed steps start with were read longest ago."""
    graphs = []
    for slot in range(nslots):
        step(slot)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(slot)
        graphs.append(g)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    return lambda i: graphs[i % nslots].replay()


def cpu_info():
    """Host CPU model name, logical CPUs and sockets (from /proc/cpuinfo)."""
    model, sockets, ncpu = "unknown", set(), 0
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "processor":
                    ncpu += 1
                elif key == "model name" and model == "unknown":
                    model = val
                elif key == "physical id":
                    sockets.add(val)
    except OSError:
        pass
    return {"model": model, "logical_cpus": ncpu or os.cpu_count(), "sockets": len(sockets) or 1}


def cpu_rate(fn, work, min_s, threads=None):
    """Rate (work per second) of fn() repeated until min_s seconds have run (at least once), with
    the oracle's parallel loops on `threads` threads (default: all); returns (rate, reps, s)."""
    import oracle
    full = oracle.num_threads()
    if threads:
        oracle.set_num_threads(threads)
    try:
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_s:
                break
    finally:
        oracle.set_num_threads(full)
    return work * reps / dt, reps, dt


def base_line(metric, value, unit, args, ms, dtype, config, higher=True):
    return {"metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": higher, "scaling": "weak",
            "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": config}


# ------------------------------------------------------------------ dense decode GEMV

def gemv_bytes(wtype, nrows, k, n):
    """Algorithmic bytes of one n-column GEMV: every weight byte once, n q8_1 columns, n fp32 rows."""
    import synth
    return nrows * synth.row_bytes(wtype, k) + n * (k // 32) * 36 + n * nrows * 4


def quant_bytes(k, n):
    return n * k * 4 + n * (k // 32) * 36


def fused_bytes(wtype, nrows, k, n):
    """Algorithmic bytes of the fused n-column call: every weight byte once, the fp32 columns,
    the fp32 outputs (the q8_1 columns never leave the workgroup)."""
    import synth
    return nrows * synth.row_bytes(wtype, k) + n * k * 4 + n * nrows * 4


def stream_read_reference(torch, M, copies, nbytes, use_graph, reps):
    """The same cold rotation read by the library's plain streaming-read kernel (one launch per
    copy, no compute): the best per-launch time over a sweep of launch shapes (256 to 3072
    workgroups of 256, 512 or 1024 threads, 4, 8 or 16 loads in flight per thread), the reference
    for what one launch reading this many bytes can reach."""
    n16 = nbytes // 16 * 16
    best = None
    for threads in (256, 512, 1024):
        for unroll, grid in ((u, g) for u in (4, 8, 16) for g in (256, 384, 512, 768, 1024, 1536, 2048, 3072)):
            if grid * threads * unroll * 16 > 8 * n16:
                continue
            out = torch.empty(grid * threads, dtype=torch.int32, device=copies[0].device)

            def batch():
                for w in copies:
                    M.qmm_debug_stream_read(w, n16, grid, threads=threads, unroll=unroll, out=out)
            t = timed_graph(torch, batch, reps, use_graph) * 1e3 / len(copies)
            if best is None or t < best[0]:
                best = (t, grid, threads, unroll)
    us, grid, threads, unroll = best
    gbps = n16 / (us * 1e-6) / 1e9
    return {"bytes": n16, "us": round(us, 3), "gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBS, 4),
            "grid": grid, "threads": threads, "unroll": unroll,
            "kernel": "stream_read_kernel (16-byte raw-buffer loads, contiguous runs per workgroup), best launch shape"}


def bench_gemv(args, torch, M, wtype, nrows, k, cols, seed, metric, name, ndistinct=6, cpu=True, cpu_s=10.0):
    import synth
    wbytes = nrows * synth.row_bytes(wtype, k)
    ncopies = max(ndistinct, -(-2 * MALL_BYTES // wbytes) + 1)
    dev = torch.device("cuda", 0)
    host_copies = [synth.weights(wtype, synth.rng_for(seed + i), nrows, k) for i in range(ndistinct)]
    copies = [torch.from_numpy(host_copies[i % ndistinct]).to(dev) for i in range(ncopies)]
    rng = synth.rng_for(seed + 100)
    xs = {n: torch.from_numpy(synth.activations(rng, n, k)).to(dev) for n in cols}
    xqs = {n: torch.empty((n, (k // 32) * 36), dtype=torch.uint8, device=dev) for n in cols}
    ys = {n: torch.empty((n, nrows), dtype=torch.float32, device=dev) for n in cols}
    for n in cols:
        M.qmm_quantize_q8_1(xs[n], out=xqs[n])
    torch.cuda.synchronize()
    use_graph = not args.no_graph
    # the calls that quantize inside the GEMV (rows of at most 96 blocks)
    fused = set() if args.unfused else fused_cols_of(k, cols)

    def step(slot):
        w = copies[slot % ncopies]
        for n in cols:
            if n in fused:
                M.qgemv_dense_f32(wtype, w, nrows, k, xs[n], n, y=ys[n])
                continue
            M.qmm_quantize_q8_1(xs[n], out=xqs[n])
            M.qgemv_dense(wtype, w, nrows, k, xqs[n], n, y=ys[n])

    run_step = capture_slots(torch, step, ncopies) if use_graph else step
    ms = contract_steps(torch, run_step, args.steps, args.warmup)
    step_bytes = sum(fused_bytes(wtype, nrows, k, n) if n in fused else gemv_bytes(wtype, nrows, k, n) +
                     quant_bytes(k, n) for n in cols)

    us, gbps, warm, literal = {}, {}, {}, {}
    for n in cols:
        def batch(n=n):
            for w in copies:
                M.qgemv_dense(wtype, w, nrows, k, xqs[n], n, y=ys[n])
        t = timed_graph(torch, batch, args.batch_reps, use_graph) * 1e3 / ncopies
        us[str(n)] = round(t, 3)
        gbps[str(n)] = round(gemv_bytes(wtype, nrows, k, n) / (t * 1e-6) / 1e9, 1)

        def warm_batch(n=n):
            for _ in range(ncopies):
                M.qgemv_dense(wtype, copies[0], nrows, k, xqs[n], n, y=ys[n])
        warm[str(n)] = round(timed_graph(torch, warm_batch, args.batch_reps, use_graph) * 1e3 / ncopies, 3)

        def lit_batch(n=n):
            for i in range(ncopies):
                M.qgemv_dense(wtype, copies[i % ndistinct], nrows, k, xqs[n], n, y=ys[n])
        literal[str(n)] = round(timed_graph(torch, lit_batch, args.batch_reps, use_graph) * 1e3 / ncopies, 3)
    fused_us = {}
    for n in sorted(fused):
        def fused_batch(n=n):
            for w in copies:
                M.qgemv_dense_f32(wtype, w, nrows, k, xs[n], n, y=ys[n])
        fused_us[str(n)] = round(timed_graph(torch, fused_batch, args.batch_reps, use_graph) * 1e3 / ncopies, 3)
    # the roofline of the GEMV launches the step runs: the fused call where the step fuses, the
    # q8_1 GEMV elsewhere (each on the cold rotation)
    tot_b = sum(fused_bytes(wtype, nrows, k, n) if n in fused else gemv_bytes(wtype, nrows, k, n) for n in cols)
    tot_us = sum(fused_us[str(n)] if n in fused else us[str(n)] for n in cols)
    achieved = tot_b / (tot_us * 1e-6) / 1e9
    floor = stream_read_reference(torch, M, copies, wbytes, use_graph, args.batch_reps)
    rec = recorded_traffic(f"gemv:{wtype}:{nrows}x{k}")
    traffic = None
    if rec and all(str(n) in rec["bytes_per_launch"] for n in cols) and \
            sorted(rec.get("fused_columns", [])) == sorted(fused):
        traffic = round(sum(rec["bytes_per_launch"][str(n)] for n in cols) / len(cols))
    parts = [f"gemv_f32_kernel at {sorted(fused)} column(s) (q8_1 formed in the kernel)"] if fused else []
    rest = [n for n in cols if n not in fused]
    if rest:
        parts.append(f"gemv_kernel at {rest} columns")
    kernels = " + ".join(parts)
    out = base_line(metric, step_bytes / (ms * 1e-3) / 1e9, "GB/s", args, ms, "int8",
                    {"workload": f"{name}, cold rotation of {ncopies} weight copies "
                                 f"({ncopies * wbytes / 1e6:.0f} MB)", "nrows": nrows, "k": k, "columns": list(cols),
                     "weight_copies": ncopies, "hip_graph": use_graph,
                     "fused_columns": sorted(fused)})
    if fused:
        out["fused_us_per_call"] = fused_us
    out.update({"us_per_call": us, "gbps_per_call": gbps, "warm_us_per_call": warm,
                f"rotation_{ndistinct}_copies_us_per_call": literal, "hbm_read_reference": floor,
                "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                             "algorithmic_bytes_per_launch": round(tot_b / len(cols)),
                             "us_per_launch": round(tot_us / len(cols), 3), "kernel": kernels}})
    if cpu and not args.no_cpu:
        out["cpu_baseline"] = cpu_gemv(wtype, host_copies[0], nrows, k, cols, seed, step_bytes, cpu_s)
    return out


def cpu_gemv(wtype, w_host, nrows, k, cols, seed, step_bytes, min_s=10.0):
    """The oracle on the same step (q8_1 of the columns and the GEMV at each column count), on all
    host threads for about min_s seconds and on one thread for about min_s / 2."""
    import oracle
    import synth
    rng = synth.rng_for(seed + 100)
    xs = {n: synth.activations(rng, n, k) for n in cols}

    def one_step():
        for n in cols:
            oracle.gemv(wtype, w_host, k, oracle.quantize_q8_1(xs[n]))
    rate, reps, dt = cpu_rate(one_step, step_bytes, min_s)
    rate1, reps1, dt1 = cpu_rate(one_step, step_bytes, min_s / 2, threads=1)
    info = cpu_info()
    return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the full step ({nrows} rows at {list(cols)} columns + q8_1 of the columns) x {reps} "
                      f"repetitions, {dt:.1f} s, {dt / reps * 1e3:.1f} ms per step",
            "one_thread": {"value": round(rate1 / 1e9, 4), "unit": "GB/s",
                           "sample": f"the same step x {reps1}, {dt1:.1f} s, {dt1 / reps1 * 1e3:.1f} ms per step"},
            "host_cpu": info["model"], "logical_cpus": info["logical_cpus"], "sockets": info["sockets"]}


# ------------------------------------------------------------------ grouped MoE decode

def grouped_bytes(hidden, inter, ngroups, m, expert_bytes):
    """Algorithmic bytes of one call: the groups' experts once, m q8_1 columns, H written and read,
    fp32 outputs."""
    nent = ngroups * m
    return ngroups * expert_bytes + m * (hidden // 32) * 36 + nent * (inter // 32) * 36 * 2 + nent * hidden * 4


def grouped_setup(torch, M):
    """Weights (expert sets in rotation), routings and buffers of the grouped decode workload;
    returns (slots, calls, call(m, slot), host weights, grid, sizes).  A slot is an (expert set,
    routing) pair: the routings of one m take disjoint experts, so the rotation over the slots
    reads nsets * nexp / ngroups distinct groups of experts (over twice the memory-side cache)
    and every call starts from HBM."""
    import numpy as np

    import synth
    nexp, hidden, inter, ngroups = 128, 2560, 1024, 16
    seed = synth.SEEDS["grouped_decode"]
    rng = synth.rng_for(seed)
    grid = synth.cb3_grid(synth.rng_for(synth.SEEDS["cb3_grid"]))
    dev = torch.device("cuda", 0)
    expert_bytes = 2 * synth.row_bytes(synth.CB3, hidden) * inter + synth.row_bytes(synth.IQ4_NL, inter) * hidden
    nroutes = nexp // ngroups                                          # disjoint routings per m
    touched = nroutes * ngroups * expert_bytes                         # distinct bytes per set
    nsets = max(2, -(-2 * MALL_BYTES // touched) + 1)                  # expert sets in rotation
    slots = [(s, r) for r in range(nroutes) for s in range(nsets)]
    host = dict(wg=np.stack([synth.cb3_weights(rng, inter, hidden) for _ in range(nexp)]),
                wu=np.stack([synth.cb3_weights(rng, inter, hidden) for _ in range(nexp)]),
                wd=np.stack([synth.iq4nl_weights(rng, hidden, inter) for _ in range(nexp)]))
    sets = [{k: torch.from_numpy(v).to(dev) for k, v in host.items()} for _ in range(nsets)]
    gd = torch.from_numpy(grid).to(dev)
    calls = {}
    for m in GROUPED_M:
        routes = synth.decode_routings(synth.rng_for(seed + m), nexp, ngroups, m, nroutes)
        x = synth.activations(synth.rng_for(seed + 100 + m), m, hidden)
        xd = torch.from_numpy(x).to(dev)
        xq = M.qmm_quantize_q8_1(xd)
        y = torch.empty((ngroups * m, hidden), dtype=torch.float32, device=dev)
        ws = torch.empty(max(16, M.qgemv_grouped_experts_workspace(inter, ngroups * m)), dtype=torch.uint8, device=dev)
        calls[m] = dict(routes=[tuple(torch.from_numpy(a).to(dev) for a in r) for r in routes],
                        x=xd, xq=xq, y=y, ws=ws, host=routes[0] + (x,))

    def call(m, slot):
        c = calls[m]
        s, r = sets[slot[0]], c["routes"][slot[1]]
        M.qgemv_grouped_experts(synth.CB3, s["wg"], s["wu"], synth.IQ4_NL, s["wd"], hidden, inter, c["xq"], r[0],
                                r[1], r[2], grid=gd, y=c["y"], ws=c["ws"])

    sizes = dict(nexp=nexp, hidden=hidden, inter=inter, ngroups=ngroups, expert_bytes=expert_bytes, nsets=nsets,
                 nroutes=nroutes, touched=touched)
    return slots, calls, call, host, grid, sizes


def bench_grouped(args, torch, M, cpu_s=10.0):
    import synth
    ms_list = GROUPED_M
    slots, calls, call, host, grid, z = grouped_setup(torch, M)
    hidden, inter, ngroups, expert_bytes, nsets, nexp = (z["hidden"], z["inter"], z["ngroups"], z["expert_bytes"],
                                                         z["nsets"], z["nexp"])
    use_graph = not args.no_graph

    def step(i):
        for m in ms_list:
            M.qmm_quantize_q8_1(calls[m]["x"], out=calls[m]["xq"])
            call(m, slots[i % len(slots)])

    run_step = capture_slots(torch, step, len(slots)) if use_graph else step
    ms = contract_steps(torch, run_step, args.steps, args.warmup)
    step_bytes = sum(grouped_bytes(hidden, inter, ngroups, m, expert_bytes) + quant_bytes(hidden, m) for m in ms_list)
    us, gbps = {}, {}
    tot_b = tot_us = 0.0
    for m in ms_list:
        def batch(m=m):
            for sl in slots:
                call(m, sl)
        t = timed_graph(torch, batch, args.batch_reps, use_graph) * 1e3 / len(slots)
        b = grouped_bytes(hidden, inter, ngroups, m, expert_bytes)
        us[str(m)] = round(t, 3)
        gbps[str(m)] = round(b / (t * 1e-6) / 1e9, 1)
        tot_b += b
        tot_us += t
    ach = tot_b / (tot_us * 1e-6) / 1e9
    rec = recorded_traffic("grouped")
    traffic = round(sum(rec["bytes_per_launch"][str(m)] for m in ms_list) / len(ms_list)) if rec else None
    out = base_line("µs/call and achieved HBM GB/s, grouped MoE decode (16 groups x m entries, 128 experts)",
                    step_bytes / (ms * 1e-3) / 1e9, "GB/s", args, ms, "int8",
                    {"workload": "grouped MoE decode: hidden 2560, 128 experts, CB3 gate/up 2560->1024, IQ4_NL down "
                                 f"1024->2560, 16 groups x m entries (m = 1/4/8); calls rotate over {len(slots)} "
                                 f"(expert set, routing) pairs, {nsets} sets x {z['nroutes']} routings with disjoint "
                                 f"experts ({nsets * z['touched'] / 1e6:.0f} MB read per rotation)",
                     "entries_per_group": list(ms_list),
                     "hip_graph": use_graph})
    out.update({"us_per_call": us, "gbps_per_call": gbps,
                "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                             "algorithmic_bytes_per_launch": round(tot_b / len(ms_list)),
                             "kernel": "gu_kernel + down_kernel (one call, m = 1/4/8)"}})
    if not args.no_cpu:
        import oracle

        def one_call(m):
            ge, go, ec, x = calls[m]["host"]
            oracle.grouped(synth.CB3, host["wg"], host["wu"], synth.IQ4_NL, host["wd"], hidden, inter,
                           oracle.quantize_q8_1(x), ge, go, ec, grid)
        rate, reps, dt = cpu_rate(lambda: [one_call(m) for m in ms_list], step_bytes, cpu_s)
        b1 = grouped_bytes(hidden, inter, ngroups, 1, expert_bytes) + quant_bytes(hidden, 1)
        rate1, reps1, dt1 = cpu_rate(lambda: one_call(1), b1, cpu_s / 2, threads=1)
        info = cpu_info()
        out["cpu_baseline"] = {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
                               "kind": "oracle", "sample": f"the full step (m = 1/4/8) x {reps}, {dt:.1f} s",
                               "one_thread": {"value": round(rate1 / 1e9, 4), "unit": "GB/s",
                                              "sample": f"the m = 1 call x {reps1}, {dt1:.1f} s"},
                               "host_cpu": info["model"], "logical_cpus": info["logical_cpus"],
                               "sockets": info["sockets"]}
    return out


# ------------------------------------------------------------------ prefill grouped expert GEMM

def prefill_setup(torch, M):
    """Weights, tokens, routing and buffers of the prefill workload; returns (call, host data, sizes)."""
    import numpy as np

    import synth
    nexp, ntok, topk, hidden, inter = 128, 8192, 8, 2560, 1024
    seed = synth.SEEDS["prefill"]
    rng = synth.rng_for(seed)
    dev = torch.device("cuda", 0)
    wg = np.stack([synth.iq4nl_weights(rng, inter, hidden) for _ in range(nexp)])
    wu = np.stack([synth.iq4nl_weights(rng, inter, hidden) for _ in range(nexp)])
    wd = np.stack([synth.q8_0_weights(rng, hidden, inter) for _ in range(nexp)])
    x16 = synth.prefill_tokens(rng, ntok, hidden)
    st, off = synth.prefill_routing(rng, ntok, nexp, topk)
    d = dict(wg=torch.from_numpy(wg).to(dev), wu=torch.from_numpy(wu).to(dev), wd=torch.from_numpy(wd).to(dev),
             x=torch.from_numpy(x16.view(np.uint16)).to(dev), st=torch.from_numpy(st).to(dev),
             off=torch.from_numpy(off).to(dev))
    nent = st.size
    y = torch.empty((nent, hidden), dtype=torch.float32, device=dev)
    ws = torch.empty(M.qgemm_prefill_experts_workspace(nexp, inter, nent), dtype=torch.uint8, device=dev)

    def call(_i=0):
        M.qgemm_prefill_experts(synth.IQ4_NL, d["wg"], d["wu"], synth.Q8_0, d["wd"], nexp, hidden, inter, d["x"],
                                d["st"], d["off"], y=y, ws=ws)

    host = dict(wg=wg, wu=wu, wd=wd, x16=x16, st=st, off=off)
    return call, host, dict(nexp=nexp, ntok=ntok, topk=topk, hidden=hidden, inter=inter, nent=nent, dev_inputs=d)


def mfma_reference(torch, M, reps):
    """Rate of the prefill GEMM's MFMA instruction in the library's register-only loop (8
    independent accumulators per wave, 4 waves per workgroup, 8 workgroups per CU, no memory):
    the rate this chip sustains for that instruction, set beside the published peak."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    grid, iters = 8 * ncu, 4000
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    M.qmm_debug_mfma_loop(grid, iters, out=out)
    ms = timed_graph(torch, lambda: M.qmm_debug_mfma_loop(grid, iters, out=out), reps, False)
    flops = grid * 4 * 8 * iters * 32 * 32 * 16 * 2
    tf = flops / (ms * 1e-3) / 1e12
    return {"tflops": round(tf, 1), "frac_of_peak": round(tf / FP16_MFMA_PEAK_TFLOPS, 4), "ms": round(ms, 3),
            "kernel": "qmm_debug_mfma_loop (v_mfma_f32_32x32x16_f16, 8 accumulators per wave, registers only)"}


def prefill_bytes(h, z):
    """Algorithmic bytes of one prefill call: every expert's weights, the tokens and the routing
    read once, H written and read once (fp16), Y written once (fp32)."""
    w = h["wg"].nbytes + h["wu"].nbytes + h["wd"].nbytes
    ids = h["st"].nbytes + h["off"].nbytes
    return int(w + h["x16"].nbytes + ids + 2 * z["nent"] * z["inter"] * 2 + z["nent"] * z["hidden"] * 4)


def bench_prefill(args, torch, M, cpu_s=10.0):
    import numpy as np

    import synth
    call, h, z = prefill_setup(torch, M)
    wg, wu, wd, x16, st, off = h["wg"], h["wu"], h["wd"], h["x16"], h["st"], h["off"]
    nexp, ntok, hidden, inter, nent = z["nexp"], z["ntok"], z["hidden"], z["inter"], z["nent"]
    use_graph = not args.no_graph
    run_step = capture_slots(torch, call, 1) if use_graph else call
    ms = contract_steps(torch, run_step, args.steps, args.warmup)
    flops = 2.0 * nent * 2 * inter * hidden + 2.0 * nent * hidden * inter
    tflops = flops / (ms * 1e-3) / 1e12
    out = base_line("µs/call and MFMA TFLOP/s, prefill grouped expert GEMM (8192 tokens x 2560, top-8 of 128)",
                    tflops, "TFLOP/s", args, ms, "fp16",
                    {"workload": "prefill grouped expert GEMM: 8192 tokens x hidden 2560, top-8 of 128 experts, "
                                 "IQ4_NL gate/up 2560->1024, Q8_0 down 1024->2560, weights converted to FP16 in registers + "
                                 "fp16 MFMA with fp32 sums",
                     "tokens": ntok, "entries": int(nent), "hip_graph": use_graph})
    rec = recorded_traffic("prefill")
    out["mfma_reference"] = mfma_reference(torch, M, args.batch_reps)
    out.update({"us_per_call": round(ms * 1e3, 2),
                "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": FP16_MFMA_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(tflops / FP16_MFMA_PEAK_TFLOPS, 4),
                             "traffic": rec["bytes_per_launch"]["call"] if rec else None,
                             "algorithmic_bytes_per_call": prefill_bytes(h, z),
                             "kernel": "schedule + pf_gateup_kernel + pf_down_kernel (one call)"}})
    if not args.no_cpu:
        import oracle

        def rows(n):
            oracle.prefill_rows(synth.IQ4_NL, wg, wu, synth.Q8_0, wd, nexp, hidden, inter, x16, st, off,
                                np.arange(n, dtype=np.int64))
        # rows of the first experts (their weights dequantized too), sized from a 32-row trial to
        # about cpu_s seconds of work on all threads; 8 rows on one thread
        t0 = time.perf_counter()
        rows(32)
        trial = time.perf_counter() - t0
        nrow = int(min(nent, max(32, 32 * cpu_s / max(trial, 1e-3))))
        rate, _, dt = cpu_rate(lambda: rows(nrow), flops / nent * nrow, 0.0)
        rate1, _, dt1 = cpu_rate(lambda: rows(8), flops / nent * 8, 0.0, threads=1)
        info = cpu_info()
        out["cpu_baseline"] = {"value": round(rate / 1e12, 6), "unit": "TFLOP/s",
                               "cores": oracle.num_threads(), "kind": "oracle",
                               "sample": f"the first {nrow} sorted rows (experts 0..{int(np.searchsorted(off, nrow, 'right')) - 1}, "
                                         f"incl. dequantizing their weights), {dt:.1f} s, as a rate per row",
                               "one_thread": {"value": round(rate1 / 1e12, 6), "unit": "TFLOP/s",
                                              "sample": f"the first 8 sorted rows, {dt1:.1f} s"},
                               "host_cpu": info["model"], "logical_cpus": info["logical_cpus"],
                               "sockets": info["sockets"]}
    return out


# ------------------------------------------------------------------ the next rows: combine, dense projections, planes

def combine_bytes(ntok, topk, hidden):
    """Algorithmic bytes of one combine: every routed row read once, the indices and weights, the
    output written once."""
    return ntok * topk * hidden * 4 + ntok * topk * 8 + ntok * hidden * 4


COMBINE_SHAPES = (("prefill_8192tok_top8", 8192, 8, None), ("decode_8tok_top16", 8, 16, 128))


def combine_setup(torch, M, rng, ntok, topk, nrows, hidden=2560):
    """Inputs of one combine workload: expert rows y, the tokens' row indices and router weights
    (the prefill shape's indices from its sorted routing, the decode shape's token-major);
    returns (call, host index, host weights, y)."""
    import synth
    dev = torch.device("cuda", 0)
    if nrows is None:
        st, _ = synth.prefill_routing(rng, ntok, 128, topk)
        idx = synth.token_positions(st, ntok, topk)
        nrows = st.size
    else:
        idx = (np.arange(topk)[None, :] * ntok + np.arange(ntok)[:, None]).astype(np.int32)
    y = torch.randn((nrows, hidden), dtype=torch.float32, device=dev)
    w = synth.router_weights(rng, ntok, topk)
    di, dw = torch.from_numpy(idx).to(dev), torch.from_numpy(w).to(dev)
    out = torch.empty((ntok, hidden), dtype=torch.float32, device=dev)
    return (lambda: M.qmm_moe_combine(y, di, dw, out=out)), idx, w, y


def bench_combine(args, torch, M, cpu_s=3.0):
    """MoE combine on the prefill workload (8192 tokens, top-8 of 128, hidden 2560: the sorted
    entry rows are 671 MB, over twice the memory-side cache, so every call reads them from HBM)
    and on the decode shape (8 tokens x 16 experts)."""
    import oracle
    import synth
    rng = synth.rng_for(synth.SEEDS["prefill"] + 10)
    res = {}
    for name, ntok, topk, nrows in COMBINE_SHAPES:
        hidden = 2560
        call, idx, w, y = combine_setup(torch, M, rng, ntok, topk, nrows, hidden)
        nrows = y.shape[0]
        # calls per graph: a replay of one graph per short call would time the host's replay rate
        per = 1 if ntok > 64 else 100

        def calls():
            for _ in range(per):
                call()
        ms = timed_graph(torch, calls, 10, not args.no_graph) / per
        b = combine_bytes(ntok, topk, hidden)
        gbps = b / (ms * 1e-3) / 1e9
        rec = recorded_traffic("combine")
        r = {"us_per_call": round(ms * 1e3, 3), "gbps": round(gbps, 1),
             "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(gbps / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": b,
                          "traffic": rec["bytes_per_launch"].get(name) if rec else None,
                          "kernel": "combine_kernel"},
             "workload": f"{ntok} tokens x top-{topk}, hidden {hidden}, {nrows} rows of y ({nrows * hidden * 4 / 1e6:.0f} MB)"}
        if not args.no_cpu:
            yh = y.cpu().numpy()
            rate, reps_c, dt = cpu_rate(lambda: oracle.moe_combine(yh, idx, w), b, cpu_s)
            r["cpu_baseline"] = {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
                                 "kind": "oracle", "sample": f"the same call x {reps_c}, {dt:.1f} s"}
        res[name] = r
        del y
    return res


def dense_specs():
    """The dense projections' matrices: (weight type, rows, seed key); K = 2560."""
    import synth
    return ((synth.IQ4_NL, 8192, "iq4nl_8192x2560"), (synth.Q8_0, 12288, "q8_0_12288x2560"))


def dense_tokens(torch, ntok, k):
    """The prompt tokens of the dense projections (binary16), host and device."""
    import synth
    x16 = synth.prefill_tokens(synth.rng_for(synth.SEEDS["prefill"] + 20), ntok, k)
    return x16, torch.from_numpy(x16.view(np.uint16)).to(torch.device("cuda", 0))


def dense_name(wt, nrows, k):
    import synth
    return f"{'iq4_nl' if wt == synth.IQ4_NL else 'q8_0'}_{nrows}x{k}_8192tok"


def dense_setup(torch, M, wt, nrows, k, key, xd):
    """Weights and output of one dense projection; returns (host weights, device weights, y,
    the fused call)."""
    import synth
    dev = torch.device("cuda", 0)
    w = synth.weights(wt, synth.rng_for(synth.SEEDS[key]), nrows, k)
    wd = torch.from_numpy(w).to(dev)
    y = torch.empty((xd.shape[0], nrows), dtype=torch.float32, device=dev)
    return w, wd, y, (lambda: M.qgemm_dense(wt, wd, nrows, k, xd, y=y))


def bench_dense(args, torch, M, cpu_s=3.0):
    """Dense prompt projections: 8192 prompt tokens through the decode workloads' matrices
    (IQ4_NL 8192 x 2560 and Q8_0 12288 x 2560), fused (weights converted to FP16 inside the
    GEMM) and in two steps (qmm_dequant_f16 with 16-byte stores, then the GEMM on FP16 weights)."""
    import oracle
    import synth
    ntok, k = 8192, 2560
    x16, xd = dense_tokens(torch, ntok, k)
    res = {}
    for wt, nrows, key in dense_specs():
        w, wd, y, fused_call = dense_setup(torch, M, wt, nrows, k, key, xd)
        w16 = torch.empty((nrows, k), dtype=torch.float16, device=wd.device)
        g = not args.no_graph
        fused = timed_graph(torch, fused_call, 10, g)
        deq = timed_graph(torch, lambda: M.qmm_dequant_f16(wt, wd, nrows, k, out=w16), 50, g)
        f16 = timed_graph(torch, lambda: M.qgemm_dense(M.QMM_F16, w16, nrows, k, xd, y=y), 10, g)
        # reference: the vendor BLAS (torch.mm on the same FP16 operands, fp32 output)
        xh = xd.view(torch.float16)
        vendor = timed_graph(torch, lambda: torch.mm(xh, w16.t(), out_dtype=torch.float32), 10, g)
        flops = 2.0 * ntok * nrows * k
        tf = flops / (fused * 1e-3) / 1e12
        deq_bytes = nrows * synth.row_bytes(wt, k) + nrows * k * 2
        name = dense_name(wt, nrows, k)
        rec = recorded_traffic("dense")
        r = {"us_per_call": round(fused * 1e3, 2), "tflops": round(tf, 1),
             "two_step": {"dequant_us": round(deq * 1e3, 2), "dequant_gbps": round(deq_bytes / (deq * 1e-3) / 1e9, 1),
                          "f16_gemm_us": round(f16 * 1e3, 2),
                          "f16_gemm_tflops": round(flops / (f16 * 1e-3) / 1e12, 1),
                          "total_us": round((deq + f16) * 1e3, 2)},
             "vendor_gemm_reference": {"us": round(vendor * 1e3, 2),
                                       "tflops": round(flops / (vendor * 1e-3) / 1e12, 1),
                                       "what": "torch.mm on the same FP16 operands, fp32 output (the vendor BLAS)"},
             "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(tf / FP16_MFMA_PEAK_TFLOPS, 4), "flops_per_launch": flops,
                          "traffic": rec["bytes_per_launch"].get(name) if rec else None,
                          "kernel": "dense_kernel (weights converted to FP16 in registers, fp16 MFMA 32x32x16)"},
             "workload": f"8192 tokens x {nrows}x{k} {'IQ4_NL' if wt == synth.IQ4_NL else 'Q8_0'}"}
        if not args.no_cpu:
            rows = np.arange(8, dtype=np.int64)
            rate, reps_c, dt = cpu_rate(lambda: oracle.dense_rows(wt, w, nrows, k, x16, rows),
                                        2.0 * 8 * nrows * k, cpu_s)
            r["cpu_baseline"] = {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
                                 "kind": "oracle", "sample": f"8 tokens (weights dequantized too) x {reps_c}, {dt:.1f} s"}
        res[name] = r
        del wd, w16, y
    return res


def planes_specs():
    """The planes GEMVs: (weight type, rows, K, column counts, seed key)."""
    import synth
    return ((synth.IQ4_NL, 8192, 2560, (1, 4, 8), "iq4nl_8192x2560"),
            (synth.Q8_0, 12288, 2560, (1, 2, 4), "q8_0_12288x2560"),
            (synth.Q8_0, 2560, 6144, (7, 8), "q8_0_2560x6144"))


def bench_planes(args, torch, M):
    """The decode GEMVs on weight planes against the same GEMVs on the GGUF blocks, each over a
    cold rotation of copies, in the same run; plus the time of one repack."""
    import synth
    dev = torch.device("cuda", 0)
    res = {}
    g = not args.no_graph
    for wt, nrows, k, cols, key in planes_specs():
        wbytes = nrows * synth.row_bytes(wt, k)
        host_w = [synth.weights(wt, synth.rng_for(synth.SEEDS[key] + i), nrows, k) for i in range(6)]
        nc = cold_copies(wbytes)
        blocks = [torch.from_numpy(host_w[i % 6]).to(dev) for i in range(nc)]
        planes = [M.qmm_pack_planes(wt, b, nrows, k) for b in blocks]
        pack_ms = timed_graph(torch, lambda: M.qmm_pack_planes(wt, blocks[0], nrows, k, out=planes[0]), 5, g)
        xq = M.qmm_quantize_q8_1(torch.from_numpy(synth.activations(synth.rng_for(7), max(cols), k)).to(dev))
        y = torch.empty((max(cols), nrows), dtype=torch.float32, device=dev)
        r = {"planes_us_per_call": {}, "blocks_us_per_call": {}, "planes_gbps": {},
             "pack_us": round(pack_ms * 1e3, 2), "weight_copies": nc}
        tot_b = tot_t = 0.0
        for n in cols:
            xn = xq[:n].contiguous()
            tp = timed_graph(torch, lambda: [M.qgemv_planes(wt, p, nrows, k, xn, n, y=y) for p in planes],
                             args.batch_reps, g) * 1e3 / nc
            tb = timed_graph(torch, lambda: [M.qgemv_dense(wt, b, nrows, k, xn, n, y=y) for b in blocks],
                             args.batch_reps, g) * 1e3 / nc
            b = gemv_bytes(wt, nrows, k, n)
            r["planes_us_per_call"][str(n)] = round(tp, 3)
            r["blocks_us_per_call"][str(n)] = round(tb, 3)
            r["planes_gbps"][str(n)] = round(b / (tp * 1e-6) / 1e9, 1)
            tot_b += b
            tot_t += tp
        ach = tot_b / (tot_t * 1e-6) / 1e9
        rec = recorded_traffic(f"planes:{wt}:{nrows}x{k}")
        r["roofline"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(ach / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_launch": round(tot_b / len(cols)),
                         "traffic": round(sum(rec["bytes_per_launch"][str(n)] for n in cols) / len(cols)) if rec else None,
                         "kernel": f"gemv_kernel on planes, columns {list(cols)}"}
        res[f"{'iq4_nl' if wt == synth.IQ4_NL else 'q8_0'}_{nrows}x{k}"] = r
        del blocks, planes
        torch.cuda.empty_cache()
    return res


INT8_MFMA_PEAK_TOPS = 5000.0
VALU_LANE_OPS_PEAK = 256 * 4 * 16 * 2.4e9     # non-packed binary32 VALU lane operations per second


def mmq_setup(torch, M):
    """The prefill workload's inputs with the MMQ-style call beside the FP16 one; returns
    (MMQ call, FP16 call, host data, sizes)."""
    import synth
    call, h, z = prefill_setup(torch, M)
    nexp, hidden, inter, nent, ntok = z["nexp"], z["hidden"], z["inter"], z["nent"], z["ntok"]
    d = z["dev_inputs"]
    y = torch.empty((nent, hidden), dtype=torch.float32, device=d["wg"].device)
    ws = torch.empty(M.qgemm_prefill_experts_q8_workspace(nexp, hidden, inter, ntok, nent), dtype=torch.uint8,
                     device=d["wg"].device)

    def mmq():
        M.qgemm_prefill_experts_q8(synth.IQ4_NL, d["wg"], d["wu"], synth.Q8_0, d["wd"], nexp, hidden, inter, d["x"],
                                   d["st"], d["off"], y=y, ws=ws)
    return mmq, call, h, z


def bench_mmq(args, torch, M, cpu_s=3.0):
    """The MMQ-style prefill (int8 MFMA on q8_1 activations, SwiGLU + q8_1 of H fused) on the
    prefill workload, beside the FP16 path on the same inputs."""
    import oracle
    import synth
    mmq, call, h, z = mmq_setup(torch, M)
    nexp, hidden, inter, nent = z["nexp"], z["hidden"], z["inter"], z["nent"]
    g = not args.no_graph
    ms = timed_graph(torch, mmq, max(args.steps, 5), g)
    ms_f16 = timed_graph(torch, call, max(args.steps, 5), g)
    flops = 2.0 * nent * 2 * inter * hidden + 2.0 * nent * hidden * inter
    tops = flops / (ms * 1e-3) / 1e12
    # the per-block rescale: one conversion and one fma per output and 32-value block
    valu_ops = 2.0 * nent * (2 * inter * (hidden // 32) + hidden * (inter // 32))
    rec = recorded_traffic("mmq")
    r = {"us_per_call": round(ms * 1e3, 2), "tops": round(tops, 1),
         "fp16_path_us_per_call": round(ms_f16 * 1e3, 2),
         "valu_floor_us": round(valu_ops / VALU_LANE_OPS_PEAK * 1e6, 1),
         "roofline": {"bound": "mfma", "achieved": round(tops, 1), "peak": INT8_MFMA_PEAK_TOPS, "unit": "TOP/s",
                      "frac": round(tops / INT8_MFMA_PEAK_TOPS, 4), "ops_per_call": flops,
                      "traffic": rec["bytes_per_launch"]["call"] if rec else None,
                      "kernel": "quantize_planes + schedule + mq_gateup_kernel + mq_down_kernel (one call)"},
         "workload": "prefill 8192 tokens x 2560, top-8 of 128 experts, IQ4_NL gate/up, Q8_0 down; q8_1 activations, "
                     "int8 MFMA, fp32 MFMA for the block scale products"}
    if not args.no_cpu:
        xq = oracle.quantize_q8_1(h["x16"].astype(np.float32))
        sl = np.arange(16, dtype=np.int64)
        exps = (np.searchsorted(h["off"], sl, side="right") - 1).astype(np.int32)

        def rows():
            oracle.grouped(synth.IQ4_NL, h["wg"], h["wu"], synth.Q8_0, h["wd"], hidden, inter, xq, exps,
                           np.arange(17, dtype=np.int32), h["st"][sl])
        rate, reps_c, dt = cpu_rate(rows, flops / nent * 16, cpu_s)
        r["cpu_baseline"] = {"value": round(rate / 1e12, 6), "unit": "TOP/s", "cores": oracle.num_threads(),
                             "kind": "oracle", "sample": f"the first 16 sorted rows x {reps_c}, {dt:.1f} s"}
    return r


def next_rows(args, torch, M):
    """The rows after the contract's workloads: MoE combine, dense prompt projections, planes,
    the MMQ-style prefill."""
    out = {}
    for name, fn in (("moe_combine", bench_combine), ("dense_prompt_projection", bench_dense),
                     ("weight_planes_gemv", bench_planes), ("mmq_prefill", bench_mmq)):
        t0 = time.perf_counter()
        out[name] = fn(args, torch, M)
        torch.cuda.empty_cache()
        progress(f"{name} done ({time.perf_counter() - t0:.0f} s)")
    return out


# ------------------------------------------------------------------ HBM traffic counters
#
# The traffic figure comes from two rocprofv3 counter runs of `--pmc-probe` (FETCH_SIZE, then
# WRITE_SIZE, kilobytes per dispatch), each scaled by what the same counter reads for a plain
# 64 MiB device copy, and is recorded by `--pmc-summary` with a digest of the sources:
#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <F> -o run -- python bench.py --pmc-probe
#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <W> -o run -- python bench.py --pmc-probe
#   python bench.py --pmc-summary <F>/run_counter_collection.csv <W>/run_counter_collection.csv

PROBE_COLS = (1, 4, 8)
# column counts whose calls take fp32 columns and form q8_1 inside the GEMV (qgemv_dense_f32):
# one column only; at 2 and 4 columns every workgroup's share of the quantization costs more
# than the quantizer launch it saves
FUSED_COLS = (1,)
GROUPED_M = (1, 4, 8)
# the Q8_0 workloads: (rows, k, columns, seed key)
Q8_SPECS = ((12288, 2560, (1, 2, 3, 4), "q8_0_12288x2560"), (2560, 6144, (7, 8), "q8_0_2560x6144"))
# the Q8_0 counter probe: those and the 512-row matrix
Q8_PROBE_SPECS = Q8_SPECS + ((512, 2560, (1,), "q8_0_tiny"),)


def fused_cols_of(k, cols):
    """Column counts the benchmark step runs as fused calls (q8_1 formed in the GEMV)."""
    return {n for n in cols if n in FUSED_COLS} if k <= 3072 else set()


def cold_copies(wbytes):
    """Weight copies of a cold rotation: more than twice the memory-side cache, at least 6."""
    return max(6, -(-2 * MALL_BYTES // wbytes) + 1)


def pmc_probe(torch, M, workload):
    """Three plain device copies of CALIB_BYTES, then one cold pass of `workload` with no graphs,
    so that every launch is a dispatch of its own: the headline GEMV once per weight copy at 1, 4
    and 8 columns (the Q8_0 GEMVs likewise at their column counts); the grouped decode once per
    rotation slot at m = 1, 4, 8; the prefill call twice (FP16 or MMQ-style); the prefill-shape
    combine three times; each dense projection twice; the planes GEMVs once per weight copy at
    their column counts."""
    import synth
    dev = torch.device("cuda", 0)
    if workload == "gemv":
        nrows, k, wt = 8192, 2560, synth.IQ4_NL
        wbytes = nrows * synth.row_bytes(wt, k)
        ncopies = -(-2 * MALL_BYTES // wbytes) + 1
        host = [synth.weights(wt, synth.rng_for(synth.SEEDS["iq4nl_8192x2560"] + i), nrows, k) for i in range(6)]
        copies = [torch.from_numpy(host[i % 6]).to(dev) for i in range(ncopies)]
        rng = synth.rng_for(synth.SEEDS["iq4nl_8192x2560"] + 100)
        xs = {n: torch.from_numpy(synth.activations(rng, n, k)).to(dev) for n in PROBE_COLS}
        xq = {n: M.qmm_quantize_q8_1(xs[n]) for n in PROBE_COLS}
        y = {n: torch.empty((n, nrows), dtype=torch.float32, device=dev) for n in PROBE_COLS}

        def run():   # the GEMV launches of the benchmark step: fused where it fuses
            for n in PROBE_COLS:
                for w in copies:
                    if n in FUSED_COLS:
                        M.qgemv_dense_f32(wt, w, nrows, k, xs[n], n, y=y[n])
                    else:
                        M.qgemv_dense(wt, w, nrows, k, xq[n], n, y=y[n])
    elif workload == "q8_0":
        wt = synth.Q8_0
        sets = []
        for nrows, k, cols, key in Q8_PROBE_SPECS:
            wbytes = nrows * synth.row_bytes(wt, k)
            host = [synth.weights(wt, synth.rng_for(synth.SEEDS[key] + i), nrows, k) for i in range(6)]
            copies = [torch.from_numpy(host[i % 6]).to(dev) for i in range(cold_copies(wbytes))]
            rng = synth.rng_for(synth.SEEDS[key] + 100)
            xs = synth.activations(rng, max(cols), k)
            xf = {n: torch.from_numpy(xs[:n].copy()).to(dev) for n in cols}
            xq = {n: M.qmm_quantize_q8_1(xf[n]) for n in cols}
            y = {n: torch.empty((n, nrows), dtype=torch.float32, device=dev) for n in cols}
            sets.append((nrows, k, cols, copies, xf, xq, y))

        def run():   # as the benchmark step: fused where it fuses
            for nrows, k, cols, copies, xf, xq, y in sets:
                for n in cols:
                    for w in copies:
                        if n in fused_cols_of(k, cols):
                            M.qgemv_dense_f32(wt, w, nrows, k, xf[n], n, y=y[n])
                        else:
                            M.qgemv_dense(wt, w, nrows, k, xq[n], n, y=y[n])
    elif workload == "grouped":
        slots, _, call, _, _, _ = grouped_setup(torch, M)

        def run():
            for m in GROUPED_M:
                for sl in slots:
                    call(m, sl)
    elif workload == "prefill":
        call, _, _ = prefill_setup(torch, M)

        def run():
            call()
            call()
    elif workload == "mmq":
        call = mmq_setup(torch, M)[0]

        def run():
            call()
            call()
    elif workload == "combine":
        _, ntok, topk, nrows = COMBINE_SHAPES[0]
        call = combine_setup(torch, M, synth.rng_for(synth.SEEDS["prefill"] + 10), ntok, topk, nrows)[0]

        def run():
            for _ in range(3):
                call()
    elif workload == "dense":
        _, xd = dense_tokens(torch, 8192, 2560)
        calls = [dense_setup(torch, M, wt, nrows, 2560, key, xd)[3] for wt, nrows, key in dense_specs()]

        def run():
            for c in calls:
                c()
                c()
    elif workload == "planes":
        sets = []
        for wt, nrows, k, cols, key in planes_specs():
            host = [synth.weights(wt, synth.rng_for(synth.SEEDS[key] + i), nrows, k) for i in range(6)]
            planes = [M.qmm_pack_planes(wt, torch.from_numpy(host[i % 6]).to(dev), nrows, k)
                      for i in range(cold_copies(nrows * synth.row_bytes(wt, k)))]
            xs = synth.activations(synth.rng_for(synth.SEEDS[key] + 100), max(cols), k)
            xq = {n: M.qmm_quantize_q8_1(torch.from_numpy(xs[:n].copy()).to(dev)) for n in cols}
            y = torch.empty((max(cols), nrows), dtype=torch.float32, device=dev)
            sets.append((wt, nrows, k, cols, planes, xq, y))

        def run():
            for wt, nrows, k, cols, planes, xq, y in sets:
                for n in cols:
                    for p in planes:
                        M.qgemv_planes(wt, p, nrows, k, xq[n], n, y=y)
    else:
        raise SystemExit(f"no counter probe for workload {workload}")
    src = torch.ones(CALIB_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    run()
    torch.cuda.synchronize()
    print(json.dumps({"probe": workload}), flush=True)


def pmc_summary(workload, fetch_csv, write_csv):
    """Per-launch HBM bytes of the probe's launches, from the two counter runs: each counter's
    kilobytes per dispatch times CALIB_BYTES over what that counter reads for the plain copies."""
    import csv
    import re

    import synth
    pattern = {"gemv": r"gemv_f32_kernel<\d+, \d+, (\d+),|gemv_kernel<\d+, false, (\d+),",
               "q8_0": r"gemv_f32_kernel<\d+, \d+, (\d+),|gemv_kernel<\d+, false, (\d+),",
               "grouped": r"(gu_kernel|down_kernel)",
               "prefill": r"(schedule_kernel|pf_gateup_kernel|pf_down_kernel)",
               "planes": r"gemv_kernel<[45], false, (\d+),",
               "combine": r"(combine_kernel)",
               "dense": r"(dense_kernel)",
               "mmq": r"(quantize_planes_kernel|schedule_kernel|mq_gateup_kernel|mq_down_kernel)"}[workload]

    def tag(name):   # the first group the pattern matched: column count or kernel name
        return next(g for g in re.search(pattern, name).groups() if g is not None)

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        ours = [r for r in rows if re.search(pattern, r["Kernel_Name"])]
        first = int(ours[0]["Dispatch_Id"])
        # the calibration copies: the large device copies just before the first launch measured
        cp = [float(r["Counter_Value"]) for r in rows
              if "copyBuffer" in r["Kernel_Name"] and int(r["Dispatch_Id"]) < first]
        calib = [v for v in cp if v >= 0.5 * max(cp)][-3:]
        return sum(calib) / len(calib), [(tag(r["Kernel_Name"]), float(r["Counter_Value"])) for r in ours]

    fcal, fk = per_kernel(fetch_csv, "FETCH_SIZE")
    wcal, wk = per_kernel(write_csv, "WRITE_SIZE")
    ff = CALIB_BYTES / 1024 / fcal
    wf = CALIB_BYTES / 1024 / wcal

    def mean(v):
        return sum(v) / len(v)

    rec = {"fetch_scale": round(ff, 4), "write_scale": round(wf, 4), "calibration_bytes": CALIB_BYTES}
    if workload in ("q8_0", "planes"):
        # dispatch order: per matrix, per column count, one launch per weight copy
        if workload == "q8_0":
            specs, prefix = [(synth.Q8_0, nrows, k, cols) for nrows, k, cols, _ in Q8_PROBE_SPECS], "gemv"
        else:
            specs, prefix = [sp[:4] for sp in planes_specs()], "planes"
        i = 0
        for wt, nrows, k, cols in specs:
            nc = cold_copies(nrows * synth.row_bytes(wt, k))
            r = dict(rec)
            fetch, write = {}, {}
            for n in cols:
                if len({g for g, _ in fk[i:i + nc]}) != 1:   # one kernel (pass width) per column count
                    raise SystemExit(f"dispatch order: expected {nc} launches of one kernel for {n} columns at {i}")
                fetch[n] = mean([v for _, v in fk[i:i + nc]])
                write[n] = mean([v for _, v in wk[i:i + nc]])
                i += nc
            fc = fused_cols_of(k, cols) if workload == "q8_0" else set()
            r["algorithmic_bytes"] = {str(n): fused_bytes(wt, nrows, k, n) if n in fc else gemv_bytes(wt, nrows, k, n)
                                      for n in cols}
            r["fused_columns"] = sorted(fc)
            r["fetch_kib"] = {str(n): round(v, 1) for n, v in fetch.items()}
            r["write_kib"] = {str(n): round(v, 1) for n, v in write.items()}
            r["bytes_per_launch"] = {str(n): round((fetch[n] * ff + write[n] * wf) * 1024) for n in cols}
            r["sources"] = list(DIGEST_SOURCES[workload])
            r["source_sha256"] = source_digest(r["sources"])
            store_traffic(f"{prefix}:{wt}:{nrows}x{k}", r)
        if i != len(fk) or len(fk) != len(wk):
            raise SystemExit(f"expected {i} GEMV dispatches, found {len(fk)} / {len(wk)}")
        return
    if workload == "gemv":
        fetch = {n: mean([v for g, v in fk if int(g) == n]) for n in PROBE_COLS}
        write = {n: mean([v for g, v in wk if int(g) == n]) for n in PROBE_COLS}
        rec["algorithmic_bytes"] = {str(n): fused_bytes(synth.IQ4_NL, 8192, 2560, n) if n in FUSED_COLS
                                    else gemv_bytes(synth.IQ4_NL, 8192, 2560, n) for n in PROBE_COLS}
        rec["fused_columns"] = list(FUSED_COLS)
        key = f"gemv:{synth.IQ4_NL}:8192x2560"
    elif workload == "grouped":
        # dispatch order: for each m, one gu_kernel and one down_kernel per expert set
        def by_m(lst):
            per_call = [lst[i][1] + lst[i + 1][1] for i in range(0, len(lst), 2)]
            c = len(per_call) // len(GROUPED_M)
            return {m: mean(per_call[i * c:(i + 1) * c]) for i, m in enumerate(GROUPED_M)}
        fetch, write = by_m(fk), by_m(wk)
        key = "grouped"
    elif workload == "combine":
        # three launches of the prefill-shape combine
        name, ntok, topk, _ = COMBINE_SHAPES[0]
        fetch, write = {name: mean([v for _, v in fk])}, {name: mean([v for _, v in wk])}
        rec["algorithmic_bytes"] = {name: combine_bytes(ntok, topk, 2560)}
        key = "combine"
    elif workload == "dense":
        # two launches per matrix, in the order of dense_specs()
        fetch, write = {}, {}
        rec["flops"] = {}
        for j, (wt, nrows, _) in enumerate(dense_specs()):
            name = dense_name(wt, nrows, 2560)
            fetch[name] = mean([v for _, v in fk[2 * j:2 * j + 2]])
            write[name] = mean([v for _, v in wk[2 * j:2 * j + 2]])
            rec["flops"][name] = 2 * 8192 * nrows * 2560
        key = "dense"
    else:
        last = "pf_down_kernel" if workload == "prefill" else "mq_down_kernel"

        def per_call(lst):
            calls, cur = [], 0.0
            for g, v in lst:
                cur += v
                if g == last:
                    calls.append(cur)
                    cur = 0.0
            return {"call": mean(calls[1:] or calls)}
        fetch, write = per_call(fk), per_call(wk)
        names = (("pf_gateup_kernel", "pf_down_kernel") if workload == "prefill"
                 else ("quantize_planes_kernel", "mq_gateup_kernel", "mq_down_kernel"))
        for name in names:
            rec[f"{name}_bytes"] = round((mean([v for g, v in fk if g == name]) * ff
                                          + mean([v for g, v in wk if g == name]) * wf) * 1024)
        key = workload
    rec["fetch_kib"] = {str(n): round(v, 1) for n, v in fetch.items()}
    rec["write_kib"] = {str(n): round(v, 1) for n, v in write.items()}
    rec["bytes_per_launch"] = {str(n): round((fetch[n] * ff + write[n] * wf) * 1024) for n in fetch}
    rec["sources"] = list(DIGEST_SOURCES[workload])
    rec["source_sha256"] = source_digest(rec["sources"])
    store_traffic(key, rec)


def store_traffic(key, rec):
    try:
        with open(TRAFFIC_FILE) as fh:
            allrec = json.load(fh)
    except (OSError, ValueError):
        allrec = {}
    allrec[key] = rec
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(allrec, fh, indent=1)
    print(json.dumps({key: rec}, indent=1))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="all",
                    choices=["all", "gemv", "tiny", "q8_0", "grouped", "prefill", "next", "mmq", "combine", "dense",
                             "planes"],
                    help="all (default): the headline GEMV line with every other workload under 'configs'")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--unfused", action="store_true", help="every GEMV call as quantizer + q8_1 GEMV")
    ap.add_argument("--batch-reps", type=int, default=5)
    ap.add_argument("--pmc-probe", action="store_true", help="launch sequence for the counter runs")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="record per-launch HBM bytes from the two counter runs (no GPU)")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.workload, *args.pmc_summary)
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): each workload is measured on one "
              "GPU's share; the design notes say how it would shard.", file=sys.stderr)
        return 2

    import torch

    import moe_expert_amd as M
    import synth

    torch.cuda.set_device(0)
    global TINY_SPEC, Q8_BENCH
    TINY_SPEC, Q8_BENCH = _bench_specs()
    if args.pmc_probe:
        pmc_probe(torch, M, args.workload)
        return 0
    if args.workload in ("gemv", "all"):
        t0 = time.perf_counter()
        out = bench_gemv(args, torch, M, synth.IQ4_NL, 8192, 2560, (1, 4, 8), synth.SEEDS["iq4nl_8192x2560"],
                         "µs/call and achieved HBM GB/s, IQ4_NL 8192x2560 GEMV at 1/4/8 columns",
                         "IQ4_NL dense decode GEMV 8192x2560 x q8_1, 1/4/8 columns")
        progress(f"headline IQ4_NL 8192x2560 GEMV done ({time.perf_counter() - t0:.0f} s)")
        if args.workload == "all":
            out["configs"] = other_configs(args, torch, M)
            out["next"] = next_rows(args, torch, M)
        print(json.dumps(out), flush=True)
    elif args.workload == "tiny":
        print(json.dumps(bench_gemv(args, torch, M, *TINY_SPEC)), flush=True)
    elif args.workload == "q8_0":
        for spec in Q8_BENCH:
            print(json.dumps(bench_gemv(args, torch, M, *spec)), flush=True)
    elif args.workload == "grouped":
        print(json.dumps(bench_grouped(args, torch, M)), flush=True)
    elif args.workload == "next":
        print(json.dumps(next_rows(args, torch, M)), flush=True)
    elif args.workload == "mmq":
        print(json.dumps(bench_mmq(args, torch, M)), flush=True)
    elif args.workload in ("combine", "dense", "planes"):
        fn = {"combine": bench_combine, "dense": bench_dense, "planes": bench_planes}[args.workload]
        print(json.dumps(fn(args, torch, M)), flush=True)
    else:
        print(json.dumps(bench_prefill(args, torch, M)), flush=True)
    return 0


def progress(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def _bench_specs():
    import synth
    tiny = (synth.Q8_0, 512, 2560, (1,), synth.SEEDS["q8_0_tiny"],
            "µs/call and achieved HBM GB/s, Q8_0 512x2560 GEMV at 1 column",
            "Q8_0 dense decode GEMV 512x2560 x q8_1, 1 column")
    q8 = [(synth.Q8_0, nrows, k, cols, synth.SEEDS[key], f"µs/call and achieved HBM GB/s, {name}", name)
          for nrows, k, cols, key, name in ((12288, 2560, (1, 2, 3, 4), "q8_0_12288x2560",
                                             "Q8_0 dense decode GEMV 12288x2560 x q8_1, 1-4 columns"),
                                            (2560, 6144, (7, 8), "q8_0_2560x6144",
                                             "Q8_0 dense decode GEMV 2560x6144 x q8_1, 7-8 columns"))]
    return tiny, q8


# keys of a workload's own line that the headline line already states
_BOILERPLATE = ("n_gpus", "higher_is_better", "scaling", "vs_baseline", "data")


def other_configs(args, torch, M):
    """The other workloads of the contract, each timed like the headline (same steps and warm-up,
    cold rotations, graphs), with a shorter oracle sample: returned as one dict per workload."""
    tiny, q8 = _bench_specs()
    runs = [("q8_0_512x2560_1col", lambda: bench_gemv(args, torch, M, *tiny, cpu_s=3.0)),
            ("q8_0_12288x2560_1to4col", lambda: bench_gemv(args, torch, M, *q8[0], cpu_s=3.0)),
            ("q8_0_2560x6144_7to8col", lambda: bench_gemv(args, torch, M, *q8[1], cpu_s=3.0)),
            ("grouped_moe_decode_128x2560x1024", lambda: bench_grouped(args, torch, M, cpu_s=4.0)),
            ("prefill_experts_8192x2560_top8", lambda: bench_prefill(args, torch, M, cpu_s=4.0))]
    out = {}
    for name, fn in runs:
        t0 = time.perf_counter()
        r = fn()
        out[name] = {k: v for k, v in r.items() if k not in _BOILERPLATE}
        torch.cuda.empty_cache()
        progress(f"{name} done ({time.perf_counter() - t0:.0f} s)")
    return out


TINY_SPEC, Q8_BENCH = None, None


if __name__ == "__main__":
    sys.exit(main())
