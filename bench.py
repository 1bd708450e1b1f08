#!/usr/bin/env python3
"""Benchmark of the CSA2 sparse-attention step on one MI355X.

Default workload ``decode_group_128k``: batch 8, 128K context, one layer group
of a Full layer plus 5 Reuse layers sharing one index set and one main K/V
cache; 16 heads x 128, int8 indexer of dim 64, blocks of 8, pool 2,048,
Top-512 plus a 128-token window.  A step is one pass of the whole path: block
pass (storing the key of the block the newest token completes), token Top-K
and the attention of all 6 layers (48 queries).  Its roofline is HBM bandwidth.
The default run also times ``prefill_8k`` (one 8,192-token prompt, a Full
layer and two window-only layers; 24,576 queries per step; MFMA roofline) and
reports it under the key ``prefill``.

Inputs are resident in HBM before timing starts.  Steps rotate over R device
replicas of the caches (each with fresh queries) so that the working set of
consecutive steps is not served from the 256 MB last-level cache.  Steps are
replayed from HIP graphs of at least 32 steps (whole cycles over the
replicas; captured through torch on the stream the library launches on), each
graph replayed once before the timed region, so host launch overhead and
first-replay costs are not timed, and the cost of a replay boundary (several
microseconds) is shared by many steps.

Per-kernel durations come from the library's own timing hook
(csa2_profile_begin): after the timed region, steps run eagerly on the same
stream with every kernel launched with HIP start/stop events, which hold that
kernel's execution interval.  ``roofline`` is the kernel of the step with the
largest time per step, its algorithmic bytes (decode) or operations (prefill)
per launch over its average duration; ``roofline_step`` is the whole step's
algorithmic work over the step time.  ``launch_floor_us`` is the time per step
of graphs as long as the timed ones holding as many near-empty launches per
step as the step has kernels.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn queries/sec + achieved HBM GB/s, decode at 128K ctx (1 GPU)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0      # dense MFMA, MI355X
INT8_PEAK_TOPS = 5000.0
KERNEL_SOURCES = ["select.hip", "attend.hip", "single.hip", "device_common.h", "internal.h"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "top_kv_selection_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """Calibrated HBM bytes per launch from committed rocprofv3 counter
    summaries, or None when there are none or the kernel sources changed since
    they were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha") != source_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


kGraphSteps = 32    # default steps per replayed graph


def run_workload(name, steps, warmup, replicas, streams, profile_rounds, cpu_seconds, graph_steps=None,
                 single=False):
    import numpy as np
    import torch

    from top_kv_selection_amd import binding as B
    from top_kv_selection_amd import pipeline
    from top_kv_selection_amd import workloads as W

    cfg = W.CONFIGS[name]
    R, NS = max(1, replicas), max(1, streams)
    if R % NS or steps % NS or warmup % NS:
        raise SystemExit("--replicas, --steps and --warmup must be multiples of --streams")
    n_queries = cfg.n_q * cfg.n_layers

    log(f"{name}: generating (seed {cfg.seed})")
    t0 = time.time()
    wl = W.generate(cfg)
    log(f"{name}: generated in {time.time() - t0:.1f}s; uploading {R} replicas")
    base = pipeline.upload(wl)
    pipeline.build_cache(base)
    dws = [base]
    for r in range(1, R):
        q_idx, q = W.fresh_queries(cfg, seed=cfg.seed * 1000 + r)
        dws.append(pipeline.replicate(base, q_idx, q))
    torch.cuda.synchronize()
    log(f"{name}: {R} replicas resident ({torch.cuda.memory_allocated() / 2**30:.1f} GiB)")

    # ---- graphs of whole steps, one set per stream (each stream owns R/NS replicas)
    def capture(fn, reps, stream=None):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for dw in reps:
                fn(dw)
        return g

    def step(dw):                       # one pass of the workload's layer groups
        pipeline.run(dw, single=single)

    for dw in dws:                      # eager pass: every launch checked once
        step(dw)
    torch.cuda.synchronize()
    RS = R // NS
    side = [torch.cuda.Stream() for _ in range(NS)]
    own = [dws[k * RS:(k + 1) * RS] for k in range(NS)]
    step_graphs = [dict() for _ in range(NS)]

    # steps per graph: whole cycles over the stream's replicas, at least
    # kGraphSteps (the order of the replicas is the same whatever the graph
    # length; a replay boundary costs several microseconds, which a graph of
    # only a few steps would add to each step)
    G = RS * max(1, -(-(graph_steps or kGraphSteps) // RS))

    def graphs_for(n):
        """Graphs for n steps per stream: graphs of G steps (cycles over the
        stream's replicas) plus one shorter tail; every new graph is replayed
        once."""
        for k in range(NS):
            for m in (G if n >= G else 0, n % G):
                if m and m not in step_graphs[k]:
                    step_graphs[k][m] = capture(step, [own[k][j % RS] for j in range(m)], side[k])
                    step_graphs[k][m].replay()
        torch.cuda.synchronize()

    def run_steps(n_total):
        n = n_total // NS
        full, rest = divmod(n, G)
        main = torch.cuda.current_stream()
        for k in range(NS):
            side[k].wait_stream(main)
            with torch.cuda.stream(side[k]):
                for _ in range(full):
                    step_graphs[k][G].replay()
                if rest:
                    step_graphs[k][rest].replay()
        for k in range(NS):
            main.wait_stream(side[k])

    graphs_for(warmup // NS)
    graphs_for(steps // NS)             # every graph of the timed region exists and has run once
    run_steps(warmup)
    torch.cuda.synchronize()
    log(f"{name}: warmup {warmup} steps done; timing {steps} steps on {NS} stream(s)")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    run_steps(steps)
    end.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / steps
    value = n_queries * steps / (ms_total / 1e3)
    log(f"{name}: {ms_per_step * 1e3:.2f} us/step, {value / 1e6:.3f} M queries/s")

    # ---- per-kernel durations: eager steps with the library's timing hook
    n_prof = profile_rounds * R
    B.csa2_profile_begin("", 64 * n_prof)
    for k in range(n_prof):
        step(dws[k % R])
    recs = B.csa2_profile_end()
    per = {}
    for kname, ms in recs:
        d = per.setdefault(kname, {"launches": 0, "ms": 0.0})
        d["launches"] += 1
        d["ms"] += ms
    n_kernels_per_step = sum(d["launches"] for d in per.values()) / n_prof

    # ---- fixed cost of the step's launches: a graph of as many near-empty
    # launches (a one-word workspace fill) per step
    tiny = torch.zeros(256, dtype=torch.uint8, device="cuda")
    n_empty = max(1, round(n_kernels_per_step))

    def empty_step(_):
        for _ in range(n_empty):
            B.csa2_workspace_init(tiny[:4])

    g_empty = capture(empty_step, list(range(G)))   # graphs as long as the step graphs
    g_empty.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(1, steps // G)
    s.record()
    for _ in range(reps):
        g_empty.replay()
    e.record()
    torch.cuda.synchronize()
    floor_us = s.elapsed_time(e) * 1e3 / (reps * G)
    log(f"{name}: {n_empty} near-empty launches per step take {floor_us:.2f} us in a graph")

    # ---- rooflines
    work = pipeline.kernel_work(cfg)   # kernel -> (unit, algorithmic amount per step)
    if single:   # one kernel does the work of the layer group's four
        work = {"k_decode_single": ("bytes", sum(a for u, a in work.values() if u == "bytes"))}
    kernels = {}
    for kname, d in sorted(per.items(), key=lambda kv: -kv[1]["ms"]):
        launches_per_step = d["launches"] / n_prof
        us_per_launch = d["ms"] * 1e3 / d["launches"]
        rec = {"us_per_launch": round(us_per_launch, 3), "launches_per_step": round(launches_per_step, 3),
               "us_per_step": round(us_per_launch * launches_per_step, 3)}
        if kname in work:
            unit, amount = work[kname]
            per_launch = amount / launches_per_step
            rate = per_launch / (us_per_launch * 1e-6)
            if unit == "bytes":
                rec.update(algorithmic_bytes_per_launch=int(per_launch), achieved_gbs=round(rate / 1e9, 1))
            else:
                rec.update({f"algorithmic_{unit}_per_launch": int(per_launch), "achieved_tops": round(rate / 1e12, 1)})
        kernels[kname] = rec
        log(f"{name}: kernel {kname}: {us_per_launch:.2f} us x {launches_per_step:g} per step")

    known = [k for k in kernels if k in work]
    if not known:
        raise SystemExit(f"no work model for the kernels of {name}: {sorted(kernels)}")
    dom = max(known, key=lambda k: kernels[k]["us_per_step"])
    unit, _ = work[dom]
    if unit == "bytes":
        ach = kernels[dom]["achieved_gbs"]
        roofline = {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(dom, name)}
        step_bytes = sum(a for u, a in work.values() if u == "bytes")
        step_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
        step = {"bound": "hbm", "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(step_gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": step_bytes}
    else:
        peak = INT8_PEAK_TOPS if unit == "int8_ops" else BF16_PEAK_TFLOPS
        ach = kernels[dom]["achieved_tops"]
        roofline = {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": peak,
                    "unit": "TOP/s" if unit == "int8_ops" else "TFLOP/s", "frac": round(ach / peak, 4),
                    "traffic": measured_traffic(dom, name)}
        int8 = sum(a for u, a in work.values() if u == "int8_ops")
        bf16 = sum(a for u, a in work.values() if u == "bf16_flops")
        ideal_us = int8 / (INT8_PEAK_TOPS * 1e6) + bf16 / (BF16_PEAK_TFLOPS * 1e6)
        step = {"bound": "mfma", "frac": round(ideal_us / (ms_per_step * 1e3), 4), "int8_ops": int8,
                "bf16_flops": bf16, "ideal_us_at_peak": round(ideal_us, 3)}

    # ---- CPU baseline: the oracle on a bounded sample of the same step
    cpu = None
    if cpu_seconds > 0:
        import oracle

        threads = oracle.default_threads()
        log(f"{name}: cpu baseline, oracle on {threads} threads for ~{cpu_seconds:.0f}s")
        n = 0
        t0 = time.time()
        if cfg.decode:
            while True:
                oracle.run_layers(wl, threads=threads)
                n += 1
                if time.time() - t0 >= cpu_seconds:
                    break
            dt = time.time() - t0
            cpu = {"value": round(n * n_queries / dt, 2), "unit": "queries/s", "cores": threads, "kind": "oracle",
                   "sample": f"{n} full steps of {name} ({n_queries} queries each) on replica 0, {dt:.1f}s"}
        else:
            rng = np.random.default_rng(0)
            rows_done = 0
            while True:
                rows = np.sort(rng.choice(cfg.n_q, min(256, cfg.n_q), replace=False))
                oracle.run_layers(wl, rows=rows, threads=threads)
                rows_done += len(rows)
                if time.time() - t0 >= cpu_seconds:
                    break
            dt = time.time() - t0
            cpu = {"value": round(rows_done * cfg.n_layers / dt, 2), "unit": "queries/s", "cores": threads,
                   "kind": "oracle",
                   "sample": f"{rows_done} random query rows of {name}, all {cfg.n_layers} layers, {dt:.1f}s"}
        log(f"{name}: cpu baseline {cpu['value']} queries/s")

    res = {
        "value": round(value, 1),
        "unit": "queries/s",
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 6),
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "config": {"workload": name, "batch": cfg.n_seq, "context": cfg.ctx, "layers": "+".join(cfg.layers),
                   "queries_per_step": n_queries, "heads": cfg.n_heads, "head_dim": cfg.head_dim,
                   "d_idx": cfg.d_idx, "block": cfg.block, "pool": cfg.pool, "top_k": cfg.top_k,
                   "window": cfg.window, "ratio": cfg.ratio, "replicas": R, "streams": NS,
                   "single_launch": bool(single),
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "roofline_step": step,
        "launch_floor_us": round(floor_us, 3),
        "kernels_per_step": round(n_kernels_per_step, 3),
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    del dws, base, own, step_graphs, g_empty
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (decode 3200, prefill 200)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (decode 320, prefill 20)")
    ap.add_argument("--replicas", type=int, default=None,
                    help="device replicas rotated over (decode 32, prefill 2: about 450 MB)")
    ap.add_argument("--streams", type=int, default=1,
                    help="independent steps in flight on separate streams (micro-batch overlap); "
                         "each stream owns replicas/streams replicas")
    ap.add_argument("--workload", default=None,
                    help="one workload only (default: decode_group_128k, plus prefill_8k under 'prefill')")
    ap.add_argument("--profile-rounds", type=int, default=2, help="eager passes over the replicas with kernel timing")
    ap.add_argument("--single-launch", action="store_true",
                    help="run Full/Reindex layer groups through csa2_layer_group_single (one launch each)")
    ap.add_argument("--graph-steps", type=int, default=None,
                    help="steps per replayed graph, rounded up to whole cycles over the replicas "
                         f"(default {kGraphSteps})")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run one plain 1 GiB device-to-device copy (calibrates rocprofv3 "
                         "FETCH_SIZE/WRITE_SIZE against a known byte count) and exit")
    args = ap.parse_args()

    if args.calibrate_copy:
        import torch
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n}))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every query's selection and attention run on one device); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from top_kv_selection_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    main_name = args.workload or "decode_group_128k"
    cfg = W.CONFIGS[main_name]
    steps = args.steps if args.steps is not None else (3200 if cfg.decode else 200)
    warmup = args.warmup if args.warmup is not None else (320 if cfg.decode else 20)
    replicas = args.replicas if args.replicas is not None else (32 if cfg.decode else 2)
    cpu_s = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    res = run_workload(main_name, steps, warmup, replicas, args.streams, args.profile_rounds, cpu_s,
                       args.graph_steps, args.single_launch)

    extra = {}
    if args.workload is None:
        pre = run_workload("prefill_8k", 200, 20, 2, 1, 4, 0.0 if args.no_cpu_baseline else 5.0)
        extra["prefill"] = pre

    metric = METRIC if cfg.decode else f"sparse-attn queries/sec + MFMA utilisation, {main_name} (1 GPU)"
    out = {
        "metric": metric,
        "value": res["value"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": res["steps"],
        "warmup": res["warmup"],
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res["dtype"],
        "data": "synthetic",
        "config": res["config"],
        "roofline": res["roofline"],
        "roofline_step": res["roofline_step"],
        "launch_floor_us": res["launch_floor_us"],
        "kernels_per_step": res["kernels_per_step"],
        "kernels": res["kernels"],
        "cpu_baseline": res["cpu_baseline"],
        **extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
