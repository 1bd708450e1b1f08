#!/usr/bin/env python3
"""Benchmark of the CSA2 sparse-attention step on one MI355X.

Default workload ``decode_group_128k``: batch 8, 128K context, one layer group
of a Full layer plus 5 Reuse layers sharing one index set and one main K/V
cache; 16 heads x 128, int8 indexer of dim 64, blocks of 8, pool 2,048,
Top-512 plus a 128-token window.  A step is one pass of the whole path: block
pass (storing the key of the block the newest token completes), token Top-K
and the attention of all 6 layers (48 queries).  Its roofline is HBM bandwidth.

``--workload prefill_8k``: one 8,192-token prompt, a Full layer and two
window-only layers (24,576 queries per step); its roofline is the MFMA peak
(int8 indexer, bf16 attention).

Inputs are resident in HBM before timing starts.  Steps rotate over R device
replicas of the caches (each with fresh queries) so that the working set of
consecutive steps is not served from the 256 MB last-level cache.  Steps are
replayed from a HIP graph (captured through torch on the stream the library
launches on), so host launch overhead is not timed.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn queries/sec + achieved HBM GB/s, decode at 128K ctx (1 GPU)"
METRIC_PREFILL = "sparse-attn queries/sec + MFMA utilisation, prefill of 8K tokens (1 GPU)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0      # dense MFMA, MI355X
INT8_PEAK_TOPS = 5000.0
KERNEL_SOURCES = {
    "index_blocks": ["select.hip", "device_common.h"],
    "topk_tokens": ["select.hip", "device_common.h"],
    "attend": ["attend.hip", "device_common.h"],
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "top_kv_selection_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or None
    when there are none or the kernel source changed since they were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


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
    ap.add_argument("--workload", default="decode_group_128k")
    ap.add_argument("--kernel-reps", type=int, default=20, help="graph replays per kernel timing")
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

    import numpy as np
    import torch

    from top_kv_selection_amd import binding as B
    from top_kv_selection_amd import pipeline
    from top_kv_selection_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = W.CONFIGS[args.workload]
    if args.steps is None:
        args.steps = 3200 if cfg.decode else 200
    if args.warmup is None:
        args.warmup = 320 if cfg.decode else 20
    if args.replicas is None:
        args.replicas = 32 if cfg.decode else 2
    R = max(1, args.replicas)
    NS = max(1, args.streams)
    if R % NS:
        raise SystemExit("--replicas must be a multiple of --streams")
    K, Wm = args.steps, args.warmup
    if K % NS or Wm % NS:
        raise SystemExit("--steps and --warmup must be multiples of --streams")
    n_queries = cfg.n_q * cfg.n_layers

    log(f"generating {cfg.name} (seed {cfg.seed})")
    t0 = time.time()
    wl = W.generate(cfg)
    log(f"generated in {time.time() - t0:.1f}s; uploading {R} replicas")
    base = pipeline.upload(wl)
    pipeline.build_cache(base)
    dws = [base]
    for r in range(1, R):
        q_idx, q = W.fresh_queries(cfg, seed=cfg.seed * 1000 + r)
        dws.append(pipeline.replicate(base, q_idx, q))
    torch.cuda.synchronize()
    log(f"{R} replicas resident ({torch.cuda.memory_allocated() / 2**30:.1f} GiB)")

    # ---- graphs of whole steps, one set per stream (each stream owns R/NS replicas)
    def capture(fn, reps, stream=None):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for dw in reps:
                fn(dw)
        return g

    for dw in dws:                      # eager pass: every launch checked once
        pipeline.run(dw)
    torch.cuda.synchronize()
    RS = R // NS
    streams = [torch.cuda.Stream() for _ in range(NS)]
    own = [dws[k * RS:(k + 1) * RS] for k in range(NS)]
    step_graphs = [dict() for _ in range(NS)]

    def graphs_for(n):
        """Graphs for n steps per stream: full cycles over the stream's replicas
        plus one shorter tail."""
        for k in range(NS):
            for m in (RS if n >= RS else 0, n % RS):
                if m and m not in step_graphs[k]:
                    step_graphs[k][m] = capture(pipeline.run, own[k][:m], streams[k])

    def run_steps(n_total):
        n = n_total // NS
        full, rest = divmod(n, RS)
        graphs_for(n)
        main = torch.cuda.current_stream()
        for k in range(NS):
            streams[k].wait_stream(main)
            with torch.cuda.stream(streams[k]):
                for _ in range(full):
                    step_graphs[k][RS].replay()
                if rest:
                    step_graphs[k][rest].replay()
        for k in range(NS):
            main.wait_stream(streams[k])

    run_steps(Wm)
    torch.cuda.synchronize()
    log(f"warmup {Wm} steps done; timing {K} steps on {NS} stream(s)")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    graphs_for(K // NS)                 # every graph the timed region needs, built before it
    torch.cuda.synchronize()
    start.record()
    run_steps(K)
    end.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / K
    value = n_queries * K / (ms_total / 1e3)
    log(f"{ms_per_step * 1e3:.2f} us/step, {value / 1e6:.3f} M queries/s")

    # ---- per-kernel launch durations (graph of R back-to-back launches each)
    lc = base.lcfg

    def k_index(dw):
        for g, grp in enumerate(dw.groups):
            if grp.q_idx is not None:
                B.csa2_index_blocks(lc, grp.q_idx, dw.q_seq, dw.q_pos, dw.k_idx, dw.k_blk, dw.blk_ids[g],
                                    dw.blk_cnt[g], dw.ws)

    def k_topk(dw):
        for g, grp in enumerate(dw.groups):
            if grp.q_idx is not None:
                B.csa2_topk_tokens(lc, grp.q_idx, dw.q_seq, dw.q_pos, dw.k_idx, dw.blk_ids[g], dw.blk_cnt[g],
                                   dw.topk[g], dw.topk_cnt[g], dw.ws)

    def k_attend(dw):
        for grp in dw.groups:
            src = grp.index_of
            B.csa2_attend_group(lc, grp.q, dw.q_seq, dw.q_pos, dw.k_main, dw.v_main, grp.k_swa, grp.v_swa,
                                cfg.swa_first, dw.topk.get(src), dw.topk_cnt.get(src), grp.out, grp.lse, dw.ws)

    if cfg.decode:
        work = pipeline.algorithmic_bytes(cfg)            # bytes per launch
    else:
        work = pipeline.algorithmic_ops(cfg)              # int8 ops / bf16 flops per launch
    kernels = {}
    for name, fn in (("index_blocks", k_index), ("topk_tokens", k_topk), ("attend", k_attend)):
        launches = len(work[name])
        if launches == 0:
            continue
        g = capture(fn, dws)
        g.replay()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(args.kernel_reps):
            g.replay()
        e.record()
        torch.cuda.synchronize()
        us = s.elapsed_time(e) * 1e3 / (args.kernel_reps * R * launches)
        per_launch = sum(work[name]) / launches
        rec = {"us_per_launch": round(us, 3), "launches_per_step": launches}
        if cfg.decode:
            rec["algorithmic_bytes_per_launch"] = int(per_launch)
            rec["achieved_gbs"] = round(per_launch / (us * 1e-6) / 1e9, 1)
            log(f"kernel {name}: {us:.2f} us/launch, {rec['achieved_gbs']} GB/s algorithmic")
        else:
            unit = "int8_ops" if name != "attend" else "bf16_flops"
            rec[f"algorithmic_{unit}_per_launch"] = int(per_launch)
            rec["achieved_tops"] = round(per_launch / (us * 1e-6) / 1e12, 1)
            log(f"kernel {name}: {us:.2f} us/launch, {rec['achieved_tops']} T{unit.split('_')[0]}/s")
        kernels[name] = rec

    dom = max(kernels, key=lambda k: kernels[k]["us_per_launch"] * kernels[k]["launches_per_step"])
    extra = {}
    if cfg.decode:
        ach = kernels[dom]["achieved_gbs"]
        roofline = {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(dom, cfg.name)}
        step_bytes = sum(sum(v) for v in work.values())
        extra = {"hbm_gbs": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                 "step_algorithmic_bytes": step_bytes}
    else:
        peak = BF16_PEAK_TFLOPS if dom == "attend" else INT8_PEAK_TOPS
        ach = kernels[dom]["achieved_tops"]
        roofline = {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": peak,
                    "unit": "TFLOP/s" if dom == "attend" else "TOP/s", "frac": round(ach / peak, 4),
                    "traffic": measured_traffic(dom, cfg.name)}
        int8_ops = sum(work["index_blocks"]) + sum(work["topk_tokens"])
        bf16_flops = sum(work["attend"])
        ideal_us = int8_ops / (INT8_PEAK_TOPS * 1e6) + bf16_flops / (BF16_PEAK_TFLOPS * 1e6)
        extra = {"step_int8_ops": int8_ops, "step_bf16_flops": bf16_flops,
                 "mfma_fraction_step": round(ideal_us / (ms_per_step * 1e3), 4)}

    # ---- CPU baseline: the oracle on a bounded sample of the same step
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        threads = oracle.default_threads()
        log(f"cpu baseline: oracle steps on {threads} threads for ~{args.cpu_seconds:.0f}s")
        n = 0
        t0 = time.time()
        if cfg.decode:
            while True:
                oracle.run_layers(wl, threads=threads)
                n += 1
                if time.time() - t0 >= args.cpu_seconds:
                    break
            dt = time.time() - t0
            cpu = {"value": round(n * n_queries / dt, 2), "unit": "queries/s", "cores": threads, "kind": "oracle",
                   "sample": f"{n} full steps of {cfg.name} ({n_queries} queries each) on replica 0, {dt:.1f}s"}
        else:
            # prefill: every layer of an evenly spaced sample of query rows
            rng = np.random.default_rng(0)
            rows_done = 0
            while True:
                rows = np.sort(rng.choice(cfg.n_q, min(256, cfg.n_q), replace=False))
                oracle.run_layers(wl, rows=rows, threads=threads)
                rows_done += len(rows)
                if time.time() - t0 >= args.cpu_seconds:
                    break
            dt = time.time() - t0
            cpu = {"value": round(rows_done * cfg.n_layers / dt, 2), "unit": "queries/s", "cores": threads,
                   "kind": "oracle",
                   "sample": f"{rows_done} random query rows of {cfg.name}, all {cfg.n_layers} layers, {dt:.1f}s"}
        log(f"cpu baseline {cpu['value']} queries/s")

    out = {
        "metric": METRIC if cfg.decode else (METRIC_PREFILL if cfg.name == "prefill_8k" else
                                             f"sparse-attn queries/sec + MFMA utilisation, {cfg.name} (1 GPU)"),
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.n_seq, "context": cfg.ctx,
                   "layers": "+".join(cfg.layers), "queries_per_step": n_queries, "heads": cfg.n_heads,
                   "head_dim": cfg.head_dim, "d_idx": cfg.d_idx, "block": cfg.block, "pool": cfg.pool,
                   "top_k": cfg.top_k, "window": cfg.window, "replicas": R, "streams": NS,
                   "parallelism": "none (1 GPU)"},
        **extra,
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
