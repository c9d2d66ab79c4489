#!/usr/bin/env python3
"""Decode-step benchmark of the paged KV-cache library on one MI355X.

One step is one decode iteration of a serving batch over a paged KV cache: the
new token of every sequence is written into its slot (reshape_and_cache), then
every query attends to its whole context through its block table
(paged_attention_decode). The default workload is the Llama-3-8B-shaped layer:
64 sequences, 32 query / 8 KV heads, head_dim 128, block_size 16, context
lengths uniform in [128, 2048], bfloat16 KV scattered over a shuffled pool of
16384 blocks. Its batches hold no shared blocks, so copy_blocks has no work in
this step; it is timed on the shared-prefix workload by the tests' cases only.

Throughput = algorithmic KV bytes read per second: sum(ctx) * Hkv * 2 * D *
bytes per element per step, over the wall time of the timed steps. Inputs are
resident in HBM before timing starts. Steps rotate over several independently
generated pools (each pool set is larger than the 256 MB Infinity Cache) so a
step does not find the previous step's KV in cache.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Prints one JSON line. ``roofline`` covers the decode kernel: algorithmic bytes
per launch over its mean duration (HIP events on the launch stream) against the
8 TB/s HBM peak. ``cpu_baseline`` times the CPU oracle on the host cores on the
first pool set (test infrastructure, never the product path).
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

METRIC = "paged decode attention KV-read HBM GB/s (% of MI355X peak); seqs/s at 8B shape"
HBM_PEAK_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def build_sets(name, rotate, dev):
    import workloads as W
    builder = W.WORKLOADS[name]
    base = {"tiny_fp32": 1001, "llama3_8b_decode": 1002, "llama_70b_decode": 1003,
            "long_context_decode": 1004, "shared_prefix_cow": 1005}[name]
    sets = []
    for i in range(rotate):
        kw = {"device": dev}
        if name != "tiny_fp32":
            kw["gen_device"] = dev
        s = builder(seed=base + 100 * i, **kw)
        W.with_append(s, seed=base + 100 * i)
        s.out = torch.empty_like(s.q)
        s.kv = s.kv_bytes()          # computed once: no device sync inside the timed loop
        sets.append(s)
        log(f"[bench] built {name} set {i}: batch {s.num_seqs}, kv bytes {s.kv_bytes()}")
    return sets


def prepare(pkv, s, graphs):
    """Bind the step's two calls once; with ``graphs`` also capture each into a HIP
    graph (append, decode) so a step costs two graph launches."""
    s.app = pkv.PreparedReshapeAndCache(s.new_k, s.new_v, s.k_cache, s.v_cache, s.slot_mapping)
    s.dec = pkv.PreparedDecode(s.out, s.q, s.k_cache, s.v_cache, s.block_tables,
                               s.context_lens, s.scale, partition_size=s.partition_size)
    s.app()
    s.dec()
    torch.cuda.synchronize()
    if graphs:
        s.g_app, s.g_dec = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(s.g_app):
            s.app()
        with torch.cuda.graph(s.g_dec):
            s.dec()
        torch.cuda.synchronize()
        s.run_app, s.run_dec = s.g_app.replay, s.g_dec.replay
    else:
        s.run_app, s.run_dec = s.app, s.dec


def run_step(s, ev=None):
    s.run_app()
    if ev is not None:
        ev[0].record()
    s.run_dec()
    if ev is not None:
        ev[1].record()


def cpu_baseline(s, seconds):
    """Time the fp64 oracle on the host cores over whole batches of set 0."""
    import numpy as np
    import oracle
    prep = oracle.PreparedAttention(s.q, s.k_cache, s.v_cache, s.block_tables, s.context_lens,
                                    s.scale)
    threads = oracle.max_threads()
    reps, t_total, want = 0, 0.0, None
    while True:
        t0 = time.perf_counter()
        res = prep(threads=threads)
        t_total += time.perf_counter() - t0
        reps += 1
        want = res if want is None else want
        if t_total >= seconds or reps >= 1000:
            break
    kv = s.kv_bytes() * reps
    got = s.out.detach().cpu().double().numpy()
    err = float(np.max(np.abs(got - want)))
    return {"value": kv / t_total / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} whole batch(es) of pool set 0 ({s.num_seqs} sequences x "
                      f"{s.num_heads} heads, fp64 walk), {t_total:.1f} s",
            "seqs_per_s": s.num_seqs * reps / t_total}, err


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_8b_decode")
    ap.add_argument("--rotate", type=int, default=4,
                    help="independent pool sets the steps cycle through")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch the prepared calls directly instead of replaying HIP graphs")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(no sharding, no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    global torch
    import torch
    import paged_kv_cache_374_amd as pkv
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    pkv.load()
    sets = build_sets(args.workload, max(1, args.rotate), dev)
    torch.cuda.synchronize()
    for s in sets:
        prepare(pkv, s, graphs=not args.eager)

    for i in range(args.warmup):
        run_step(sets[i % len(sets)])
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    kv_total = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        s = sets[i % len(sets)]
        run_step(s, evs[i])
        kv_total += s.kv
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(stop)
    ms = max(gpu_ms, 1e-9)
    dec_ms = [a.elapsed_time(b) for a, b in evs]
    dec_mean = sum(dec_ms) / len(dec_ms)
    dec_sorted = sorted(dec_ms)
    kv_per_launch = kv_total / args.steps
    achieved = kv_per_launch / (dec_mean * 1e-3) / 1e9
    value = kv_total / (ms * 1e-3) / 1e9
    s0 = sets[0]
    seqs_per_s = s0.num_seqs * args.steps / (ms * 1e-3)

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline: oracle on the host cores")
        # the last step that used set 0 left its output in set 0's buffer
        cpu, parity = cpu_baseline(s0, args.cpu_seconds)

    elt = s0.q.element_size()
    dname = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[s0.dtype]
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dname,
        "data": "synthetic",
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "seqs_per_s": round(seqs_per_s, 1),
        "config": {
            "workload": s0.name,
            "batch": s0.num_seqs,
            "num_heads": s0.num_heads,
            "num_kv_heads": s0.num_kv_heads,
            "head_dim": s0.head_dim,
            "block_size": s0.block_size,
            "num_blocks": s0.num_blocks,
            "kv_dtype": dname,
            "element_bytes": elt,
            "mean_context": round(float(s0.context_lens.float().mean()), 1),
            "kv_bytes_per_step": int(kv_per_launch),
            "pool_sets": len(sets),
            "step": "reshape_and_cache(new token) + paged_attention_decode",
            "launch": "eager" if args.eager else "hip_graph",
            "wall_s_timed": round(wall, 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "paged_attention_decode",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "launch_us_mean": round(dec_mean * 1e3, 3),
            "launch_us_p10": round(dec_sorted[len(dec_sorted) // 10] * 1e3, 3),
            "launch_us_p90": round(dec_sorted[(9 * len(dec_sorted)) // 10] * 1e3, 3),
        },
        "cpu_baseline": cpu,
    }
    if parity is not None:
        line["parity_max_abs_err_vs_oracle"] = parity
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
