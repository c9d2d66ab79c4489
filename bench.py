#!/usr/bin/env python3
"""Decode-step benchmark of the paged KV-cache library on one MI355X.

One step is one decode iteration of a serving batch over a paged KV cache: the
new token of every sequence is written into its slot, then every query attends to
its whole context through its block table. By default the step is the fused call
paged_attention_decode_append (one kernel); --unfused runs it as
reshape_and_cache + paged_attention_decode. The default workload is the
Llama-3-8B-shaped layer: 64 sequences, 32 query / 8 KV heads, head_dim 128,
block_size 16, context lengths uniform in [128, 2048], bfloat16 KV scattered over a
shuffled pool of 16384 blocks. Its batches hold no shared blocks, so copy_blocks has no work in
this step; it is timed on the shared-prefix workload by the tests' cases only.

Throughput = algorithmic KV bytes read per second: sum(ctx) * Hkv * 2 * D *
bytes per element per step, over the wall time of the timed steps. Inputs are
resident in HBM before timing starts. Steps rotate over several independently
generated pools (each pool set is larger than the 256 MB Infinity Cache) so a
step does not find the previous step's KV in cache.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Workloads with several query tokens per sequence (llama3_8b_verify4: 4 draft tokens
to verify; prefill_chunk512: 512-token prefill chunks) run reshape_and_cache of the
chunk tokens, then paged_attention_chunk. A chunk workload whose arithmetic intensity
exceeds the MI355X ridge point (2.5 PFLOP/s bf16 dense / 8 TB/s) is priced against
the matrix-core peak instead of HBM.

Prints one JSON line. ``roofline`` covers the decode kernel: algorithmic bytes
per launch over its mean duration (HIP events on the launch stream) against the
8 TB/s HBM peak; where sequences share blocks, the distinct bytes instead (the
logical rate is kept beside it). ``roofline.gather_ceiling`` is the bandwidth probe
(pkv_read_tiles) on exactly the tiles the decode reads, best of a sweep of launch
shapes, and the decode's fraction of it. ``step_us`` is the p10/p50/p90 of single
steps. ``cpu_baseline`` times the CPU oracle on the host cores on the first pool set
(test infrastructure, never the product path), on all threads and, for the 8B and
tiny cases, on one; it records the CPU model and socket count.

    python bench.py --workload gather_ceiling   # the probe on its own
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
MFMA_BF16_PEAK_TFLOPS = 2500.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def build_sets(name, rotate, dev):
    import workloads as W
    builder = W.WORKLOADS[name]
    base = {"tiny_fp32": 1001, "llama3_8b_decode": 1002, "llama3_8b_decode_fp8": 1002,
            "llama3_8b_verify4": 1002, "prefill_chunk512": 1006,
            "llama_70b_decode": 1003, "long_context_decode": 1004,
            "shared_prefix_cow": 1005, "skewed_decode": 1007}[name]
    sets = []
    for i in range(rotate):
        kw = {"device": dev}
        if name != "tiny_fp32":
            kw["gen_device"] = dev
        s = builder(seed=base + 100 * i, **kw)
        W.with_append(s, seed=base + 100 * i)
        s.out = torch.empty_like(s.q)
        s.kv = s.kv_bytes()          # computed once: no device sync inside the timed loop
        s.flops = chunk_flops(s) if s.query_start is not None else 0
        # distinct physical blocks the decode reads (whole blocks), for batches that
        # share prefix blocks between sequences
        bs, tb = s.block_size, s.block_tables.cpu()
        used = {int(tb[b, j]) for b, n in enumerate(s.context_lens.cpu().tolist())
                for j in range((n + bs - 1) // bs)}
        s.kv_unique = len(used) * s.num_kv_heads * 2 * bs * s.head_dim * \
            s.k_cache.element_size()
        sets.append(s)
        log(f"[bench] built {name} set {i}: batch {s.num_seqs}, kv bytes {s.kv_bytes()}")
    return sets


def chunk_flops(s):
    """Algorithmic FLOPs of one chunk attention call: every query row (token, head)
    does 4 * D per context token it sees (QK and PV multiply-adds)."""
    qs = s.query_start.cpu().tolist()
    ctx = s.context_lens.cpu().tolist()
    seen = 0
    for b, n in enumerate(ctx):
        T = qs[b + 1] - qs[b]
        for j in range(T):
            seen += max(0, n - T + j + 1)
    return seen * s.num_heads * 4 * s.head_dim


def older_tokens_to_setup(pkv, s):
    """A batch whose append holds several tokens per sequence (the shared-prefix
    batch writes every token placed after the fork): the tokens before each
    sequence's newest are written once here, untimed, as earlier decode steps would
    have written them. The timed step appends only the newest token of each sequence,
    the one at position ctx - 1."""
    bs = s.block_size
    tables = s.block_tables.cpu().tolist()
    ctx = s.context_lens.cpu().tolist()
    slots = s.slot_mapping.cpu().tolist()
    where = {slot: t for t, slot in enumerate(slots)}
    newest = [where[tables[b][(n - 1) // bs] * bs + (n - 1) % bs] for b, n in enumerate(ctx)]
    keep = set(newest)
    older = torch.tensor([t for t in range(len(slots)) if t not in keep], device=s.q.device)
    newest = torch.tensor(newest, device=s.q.device)
    rows = (s.new_k[older].contiguous(), s.new_v[older].contiguous(), s.k_cache, s.v_cache,
            s.slot_mapping[older].contiguous())
    if s.kv_scales is not None:
        pkv.reshape_and_cache_fp8(*rows, *s.kv_scales)
    else:
        pkv.reshape_and_cache(*rows)
    s.new_k = s.new_k[newest].contiguous()
    s.new_v = s.new_v[newest].contiguous()
    s.slot_mapping = s.slot_mapping[newest].contiguous()
    torch.cuda.synchronize()


def prepare(pkv, s, graphs, fused, grouped=True):
    """Bind the step once: by default the fused call (append at each context end, then
    decode: one kernel on the matrix-core paths); with ``fused`` false the two calls
    reshape_and_cache + paged_attention_decode. A batch whose sequences share prefix
    blocks uses the grouped decode unless ``grouped`` is false. ``s.dec`` is the call
    that carries the decode kernels. With ``graphs`` the step is captured into one HIP
    graph, so a step is one graph launch."""
    copy = None
    if s.copy_pairs is not None and s.copy_pairs.numel() > 0:
        copy = pkv.PreparedCopyBlocks([s.k_cache, s.v_cache], s.copy_pairs)
        copy()                       # copy-on-write before any write after the fork
        # Repeating the copies in every step is harmless only while no written token
        # sits in a copied block, i.e. when the prefix ends on a block boundary.
        if s.extra.get("prefix_tokens", 0) % s.block_size != 0:
            copy = None
    if s.query_start is not None:
        # append the chunk tokens' K/V, then attend with every chunk token
        s.fused = False
        if s.kv_scales is not None:
            def app(s=s):
                pkv.reshape_and_cache_fp8(s.new_k, s.new_v, s.k_cache, s.v_cache,
                                          s.slot_mapping, *s.kv_scales)
        else:
            app = pkv.PreparedReshapeAndCache(s.new_k, s.new_v, s.k_cache, s.v_cache,
                                              s.slot_mapping)
        ks, vs = s.kv_scales if s.kv_scales is not None else (None, None)
        s.dec = pkv.PreparedChunk(s.out, s.q, s.k_cache, s.v_cache, s.block_tables,
                                  s.context_lens, s.query_start, s.scale, s.max_query_len,
                                  k_scale=ks, v_scale=vs)
        finish_prepare(s, [app, s.dec], graphs)
        return
    if s.new_k.shape[0] != s.num_seqs:
        older_tokens_to_setup(pkv, s)
    s.fused = fused
    ks, vs = s.kv_scales if s.kv_scales is not None else (None, None)
    if grouped and s.kv_unique < 0.98 * s.kv:
        # sequences share prefix blocks: the grouped decode reads each shared block once
        # per group (two kernels: the groups' prefixes, then each sequence's own
        # blocks). The groups come from the block tables, derived once on the host
        # before any timing, as a scheduler would when it forks the samples.
        s.groups = pkv.prefix_groups(s.block_tables, s.context_lens, s.block_size)
        s.dec = pkv.PreparedGroupedDecode(s.out, s.q, s.k_cache, s.v_cache, s.block_tables,
                                          s.context_lens, s.scale, s.groups,
                                          new_k=s.new_k if s.fused else None,
                                          new_v=s.new_v if s.fused else None,
                                          k_scale=ks, v_scale=vs)
        calls = [s.dec]
        if not s.fused:
            if s.kv_scales is not None:
                def app(s=s):
                    pkv.reshape_and_cache_fp8(s.new_k, s.new_v, s.k_cache, s.v_cache,
                                              s.slot_mapping, *s.kv_scales)
            else:
                app = pkv.PreparedReshapeAndCache(s.new_k, s.new_v, s.k_cache, s.v_cache,
                                                  s.slot_mapping)
            calls = [app, s.dec]
    elif s.fused:
        s.dec = pkv.PreparedDecode(s.out, s.q, s.k_cache, s.v_cache, s.block_tables,
                                   s.context_lens, s.scale, partition_size=s.partition_size,
                                   new_k=s.new_k, new_v=s.new_v, k_scale=ks, v_scale=vs)
        calls = [s.dec]
    else:
        if s.kv_scales is not None:
            def app(s=s):
                pkv.reshape_and_cache_fp8(s.new_k, s.new_v, s.k_cache, s.v_cache,
                                          s.slot_mapping, *s.kv_scales)
        else:
            app = pkv.PreparedReshapeAndCache(s.new_k, s.new_v, s.k_cache, s.v_cache,
                                              s.slot_mapping)
        s.dec = pkv.PreparedDecode(s.out, s.q, s.k_cache, s.v_cache, s.block_tables,
                                   s.context_lens, s.scale, partition_size=s.partition_size,
                                   k_scale=ks, v_scale=vs)
        calls = [app, s.dec]
    if copy is not None:
        calls.insert(0, copy)
    finish_prepare(s, calls, graphs)


def finish_prepare(s, calls, graphs):
    """Bind s.run to the step's calls, optionally captured in one HIP graph."""
    def run(calls=calls):
        for c in calls:
            c()
    run()
    torch.cuda.synchronize()
    if graphs:
        s.g_step = torch.cuda.CUDAGraph()
        with torch.cuda.graph(s.g_step):
            run()
        torch.cuda.synchronize()
        s.run = s.g_step.replay
    else:
        s.run = run


def time_decode_kernel(sets, graphs, per_set=4, reps=10):
    """Mean duration of one launch of the decode kernel (the fused call by default):
    back-to-back calls over the rotating pool sets (captured in one graph with
    --graphs), bracketed by HIP events on the launch stream. Repeated fused calls
    rewrite the same rows into the same slots. Returns microseconds."""
    order = [s for _ in range(per_set) for s in sets]
    if graphs:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in order:
                s.dec()
        torch.cuda.synchronize()
        launch = g.replay
    else:
        def launch():
            for s in order:
                s.dec()
    launch()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        launch()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * len(order))


def cpu_baseline(s, seconds, one_thread_seconds=0.0):
    """Time the fp64 oracle on the host cores over whole batches of set 0."""
    import numpy as np
    import oracle
    prep = oracle.PreparedAttention(s.q, s.k_cache, s.v_cache, s.block_tables, s.context_lens,
                                    s.scale, kv_scales=s.kv_scales)
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
    res = {"value": kv / t_total / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"{reps} whole batch(es) of pool set 0 ({s.num_seqs} sequences x "
                     f"{s.num_heads} heads, fp64 walk), {t_total:.1f} s",
           "seqs_per_s": s.num_seqs * reps / t_total}
    if one_thread_seconds > 0:
        # the same walk on one host thread, whole batches for a bounded time
        reps1, t1 = 0, 0.0
        while t1 < one_thread_seconds and reps1 < 1000:
            t0 = time.perf_counter()
            prep(threads=1)
            t1 += time.perf_counter() - t0
            reps1 += 1
        res["value_1thread"] = s.kv_bytes() * reps1 / t1 / 1e9
        res["seqs_per_s_1thread"] = s.num_seqs * reps1 / t1
        res["sample_1thread"] = f"{reps1} whole batch(es) of pool set 0 on 1 thread, {t1:.1f} s"
    res.update(cpu_description())
    return res, err


def cpu_baseline_tiny():
    """The oracle on the tiny float32 case (4 sequences, contexts 7..100, block size 4):
    sequences per second on all host threads and on one."""
    import oracle
    import workloads as W
    s = W.tiny_fp32(device="cpu", gen_device="cpu")
    prep = oracle.PreparedAttention(s.q, s.k_cache, s.v_cache, s.block_tables, s.context_lens,
                                    s.scale)
    out = {}
    for label, threads in (("all", oracle.max_threads()), ("1thread", 1)):
        reps, tt = 0, 0.0
        while tt < 0.5:
            t0 = time.perf_counter()
            prep(threads=threads)
            tt += time.perf_counter() - t0
            reps += 1
        out[f"seqs_per_s_{label}"] = round(s.num_seqs * reps / tt, 1)
    out["sample"] = f"tiny float32 batch (4 sequences, contexts 7/16/33/100), 0.5 s per setting"
    return out


def cpu_baseline_chunk(s, seconds, mfma_bound):
    """Time the fp64 chunk oracle on the host cores, one sequence of set 0 at a time
    (a bounded sample of the batch), and check those rows against the GPU output."""
    import numpy as np
    import torch
    import oracle
    qs = s.query_start.cpu()
    kc, vc = s.k_cache.cpu(), s.v_cache.cpu()
    tables, ctx = s.block_tables.cpu(), s.context_lens.cpu()
    got_all = s.out.detach().cpu().double().numpy()
    t_total, flops, kv, err, done = 0.0, 0, 0, 0.0, 0
    threads = oracle.max_threads()
    elt = s.k_cache.element_size()
    for b in range(s.num_seqs):
        r0, r1 = int(qs[b]), int(qs[b + 1])
        n, T = int(ctx[b]), r1 - r0
        sub_qs = torch.tensor([0, T], dtype=torch.int32)
        t0 = time.perf_counter()
        want = oracle.paged_attention_chunk(s.q[r0:r1].cpu(), kc, vc, tables[b:b + 1],
                                            ctx[b:b + 1], sub_qs, s.scale,
                                            kv_scales=s.kv_scales, threads=threads)
        t_total += time.perf_counter() - t0
        err = max(err, float(np.max(np.abs(got_all[r0:r1] - want))) if T else 0.0)
        flops += sum(max(0, n - T + j + 1) for j in range(T)) * s.num_heads * 4 * s.head_dim
        kv += n * s.num_kv_heads * 2 * s.head_dim * elt
        done += 1
        if t_total >= seconds:
            break
    value = flops / t_total / 1e12 if mfma_bound else kv / t_total / 1e9
    return {"value": value, "unit": "TFLOP/s" if mfma_bound else "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} of {s.num_seqs} sequences of pool set 0 (all their query "
                      f"rows, fp64 walk), {t_total:.1f} s"}, err


# Launch shapes the gather probe sweeps: workgroups of four waves, tiles in flight per wave.
GATHER_SHAPES = [(wg, u) for wg in (256, 512, 1024, 2048) for u in (1, 2, 4)]


def decode_tiles(s):
    """Byte offsets, in a [2, num_blocks, Hkv, bs, D] K-then-V pool, of the tiles the
    decode reads: for every (sequence, KV head), its K and V tile of each block, in
    block order (the layout and the scattered physical placement of the workload)."""
    NB, H, bs, D = s.k_cache.shape
    tile = bs * D * s.k_cache.element_size()
    tb, ctx = s.block_tables.cpu().to(torch.int64), s.context_lens.cpu().tolist()
    parts = []
    for b, n in enumerate(ctx):
        nb = (n + bs - 1) // bs
        if nb == 0:
            continue
        t = tb[b, :nb][None, :] * H + torch.arange(H)[:, None]        # [H, nb]
        parts.append(torch.stack([t, t + NB * H], dim=-1).reshape(-1))  # K, V per block
    return torch.cat(parts) * tile, tile


def gather_ceiling(pkv, sets, reps=4):
    """The bandwidth probe on exactly the tiles the decode reads (per pool set, K and V
    copied into one pool of the same layout), swept over GATHER_SHAPES: returns the best
    rate in GB/s, its shape and the whole sweep. Bytes are whole tiles, as the decode
    fetches them."""
    dev = sets[0].q.device
    preps = []
    for s in sets:
        kv = torch.empty((2,) + tuple(s.k_cache.shape), dtype=s.k_cache.dtype, device=dev)
        kv[0].copy_(s.k_cache)
        kv[1].copy_(s.v_cache)
        off, tile = decode_tiles(s)
        preps.append((kv, off.to(dev), tile))
    sink = torch.empty(max(w for w, _ in GATHER_SHAPES) * 256, dtype=torch.int32, device=dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sweep = []
    for wg, u in GATHER_SHAPES:
        def run():
            for kv, off, tile in preps:
                pkv.read_tiles(kv, off, tile, wg, u, sink)
        run()
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            run()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (reps * len(preps))
        nbytes = sum(off.numel() * tile for _, off, tile in preps) / len(preps)
        sweep.append({"workgroups": wg, "tiles_in_flight": u, "us": round(us, 3),
                      "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)})
    del preps
    best = max(sweep, key=lambda r: r["gbs"])
    return best, sweep


def cpu_description():
    """CPU model and socket count of the host (lscpu, else /proc/cpuinfo)."""
    import subprocess
    model, sockets = None, None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            k, _, v = line.partition(":")
            if k.strip() == "Model name":
                model = v.strip()
            elif k.strip() == "Socket(s)":
                sockets = int(v.strip()) if v.strip().isdigit() else v.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    if model is None:
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
    return {"cpu_model": model, "sockets": sockets, "logical_cpus": os.cpu_count()}


CALIB_PAIRS, CALIB_BLOCK_BYTES = 4096, 8 * 16 * 128 * 2


def calibrate(pkv, dev):
    """copy_blocks over CALIB_PAIRS distinct 32 KiB blocks: reads and writes exactly
    CALIB_PAIRS * CALIB_BLOCK_BYTES bytes per call; rocprofv3's FETCH_SIZE /
    WRITE_SIZE readings of this kernel give the counters' byte scale."""
    pool = torch.zeros(2 * CALIB_PAIRS, 8, 16, 128, dtype=torch.bfloat16, device=dev)
    pairs = torch.stack([torch.arange(CALIB_PAIRS), torch.arange(CALIB_PAIRS) + CALIB_PAIRS],
                        dim=1).to(torch.int32).to(dev)
    for _ in range(5):
        pkv.copy_blocks(pool, pairs)
    torch.cuda.synchronize()
    log(f"[bench] calibration: copy_blocks moved {CALIB_PAIRS * CALIB_BLOCK_BYTES} bytes "
        f"read + write per call")


def traffic_per_launch(workload):
    """Calibrated HBM bytes per decode launch from the committed rocprofv3 counter
    summary, if it was measured on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}.traffic.json")
    try:
        from paged_kv_cache_374_amd.rocprof_summary import sources_sha
        with open(path) as f:
            rec = json.load(f)
        if rec.get("source_sha") != sources_sha():
            return None
        return round(float(rec["traffic_bytes_per_launch"]))
    except (OSError, ValueError, KeyError):
        return None


HOST_LINK_PEAK_GBS = 63.0   # PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes x 128/130


def bench_swap(args, pkv, dev):
    """Swap step on the 8B batch's pool layout (8 KV heads x 16 x 128, bf16: 32 KiB per
    block per pool): 512 blocks of the K and of the V pool out to a pinned host pool,
    then 512 other blocks back in; four launches, whole-block copies."""
    import numpy as np
    import oracle
    shape = (8, 16, 128)
    n_gpu, n_host, n = 16384, 1024, 512
    g = torch.Generator(device=dev).manual_seed(1007)
    pools = [torch.randn((n_gpu,) + shape, generator=g, device=dev).to(torch.bfloat16)
             for _ in range(2)]
    hosts = [torch.zeros((n_host,) + shape, dtype=torch.bfloat16).pin_memory()
             for _ in range(2)]
    gc = torch.Generator().manual_seed(1008)
    perm = torch.randperm(n_gpu, generator=gc)
    out_pairs = torch.stack([perm[:n], torch.arange(n)], 1).to(torch.int32).to(dev)
    in_pairs = torch.stack([torch.arange(n, 2 * n), perm[n:2 * n]], 1).to(torch.int32).to(dev)
    calls = [pkv.PreparedSwapBlocks(h, p, out_pairs) for p, h in zip(pools, hosts)] + \
            [pkv.PreparedSwapBlocks(p, h, in_pairs) for p, h in zip(pools, hosts)]
    block = int(np.prod(shape)) * 2
    step_bytes = 4 * n * block

    def run():
        for c in calls:
            c()
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(args.steps):
        run()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = a.elapsed_time(b)
    value = step_bytes * args.steps / (ms * 1e-3) / 1e9
    # one launch (the K pool's swap-out) on its own, back to back
    a.record()
    for _ in range(20):
        calls[0]()
    b.record()
    torch.cuda.synchronize()
    one_us = a.elapsed_time(b) * 1e3 / 20
    achieved = n * block / (one_us * 1e-6) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's block copy on the host: swap-out of the K pool's 512 blocks
        src, host = pools[0].cpu(), hosts[0].clone()
        pairs = out_pairs.cpu()
        reps, tt = 0, 0.0
        while tt < min(args.cpu_seconds, 5.0):
            t1 = time.perf_counter()
            oracle.swap_blocks(host, src, pairs)
            tt += time.perf_counter() - t1
            reps += 1
        cpu = {"value": reps * n * block / tt / 1e9, "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{reps} swap-outs of {n} blocks (host memcpy), {tt:.1f} s"}
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "swap_blocks_8b", "block_bytes": block,
                   "blocks_per_step": 4 * n, "bytes_per_step": step_bytes,
                   "step": "swap_blocks: K and V pools, 512 blocks out to pinned host "
                           "memory, 512 other blocks in",
                   "launch": "direct (four calls per step)", "wall_s_timed": round(wall, 4)},
        "roofline": {"bound": "host link", "kernel": "swap_blocks (swap-out)",
                     "achieved": round(achieved, 2), "peak": HOST_LINK_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HOST_LINK_PEAK_GBS, 4),
                     "traffic": None, "launch_us_mean": round(one_us, 3),
                     "launch_timing": "20 back-to-back swap-outs, HIP events"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_gather(args, pkv, dev):
    """The gather ceiling on its own: the bandwidth probe on exactly the tiles the
    8B-shaped decode reads (four pool sets), swept over launch shapes."""
    sets = build_sets("llama3_8b_decode", max(1, args.rotate), dev)
    torch.cuda.synchronize()
    best, sweep = gather_ceiling(pkv, sets, reps=max(4, args.steps // len(sets)))
    nbytes = sum(decode_tiles(s)[0].numel() * decode_tiles(s)[1] for s in sets) / len(sets)
    line = {
        "metric": METRIC, "value": best["gbs"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": 1, "ms_per_step": round(best["us"] / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gather_ceiling", "tiles_per_launch": int(nbytes // 4096),
                   "bytes_per_launch": int(nbytes), "tile_bytes": 4096, "pool_sets": len(sets),
                   "step": "pkv_read_tiles over the K and V tiles of the 8B-shaped decode "
                           "batch (no arithmetic)"},
        "roofline": {"bound": "hbm", "kernel": "read_tiles", "achieved": best["gbs"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(best["gbs"] / HBM_PEAK_GBS, 4), "traffic": None,
                     "launch_us_mean": best["us"], "best_shape": best, "sweep": sweep},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bench_block_manager(args):
    """Host block manager in a serving loop on the 8B pool (16384 blocks of 16 tokens):
    32 prompts of 2040 tokens with token ids (prefix cache on), each forked into 8
    samples (so the first decoded token of 7 samples copies the shared partial block),
    then decode steps that append one token to all 256 sequences and rebuild the block
    tables the attention call takes. Times the C++ manager; the CPU baseline runs the
    same loop on the Python oracle for a few steps."""
    import random
    import numpy as np
    import oracle.blockmgr as obm
    from paged_kv_cache_374_amd.blocks import BlockManager

    nb, bs, prompts, samples, plen = 16384, 16, 32, 8, 2040
    steps = max(1, args.steps)
    rng = random.Random(1009)
    order = rng.sample(range(nb), nb)
    toks = [[rng.randrange(32000) for _ in range(plen)] for _ in range(prompts)]

    def setup(BM):
        bm = BM(nb, bs, order)
        sids = []
        for p in range(prompts):
            base = p * samples
            bm.add_sequence(base, plen, toks[p])
            sids.append(base)
            for s in range(1, samples):
                bm.fork(base, base + s)
                sids.append(base + s)
        return bm, sids

    def run(bm, sids, n, batched):
        width = (plen + n + bs - 1) // bs
        appends = 0
        sid_arr = np.asarray(sids, dtype=np.int64)
        for i in range(n):
            t = (i * 7 + np.arange(len(sids), dtype=np.int32)) % 32000
            if batched:
                placed, _, _ = bm.append_tokens(sid_arr, t)
            else:
                for sid, tok in zip(sids, t):
                    bm.append_token(sid, tok)
                placed = len(sids)
            appends += placed
            bm.build_tables(sid_arr, width)
        return appends

    bm, sids = setup(BlockManager)
    run(bm, sids, 2, True)                         # warm-up on a throwaway manager
    bm, sids = setup(BlockManager)
    t0 = time.perf_counter()
    appends = run(bm, sids, steps, True)
    dt = time.perf_counter() - t0
    value = appends / dt
    cpu = None
    if not args.no_cpu_baseline:
        om, osids = setup(obm.BlockManager)
        n_cpu = max(1, min(steps, 8))
        t1 = time.perf_counter()
        a_cpu = run(om, osids, n_cpu, False)
        tc = time.perf_counter() - t1
        cpu = {"value": a_cpu / tc, "unit": "appends/s", "cores": 1, "kind": "oracle",
               "sample": f"{n_cpu} decode steps of the same loop (Python oracle), {tc:.1f} s"}
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "appends/s", "n_gpus": 1,
        "steps": steps, "warmup": 2, "ms_per_step": round(dt * 1e3 / steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": "block_manager_serving", "num_blocks": nb, "block_size": bs,
                   "sequences": len(sids), "prompt_tokens": plen,
                   "step": "append_tokens(256 sequences) + build_tables (host)",
                   "wall_s_timed": round(dt, 4)},
        "roofline": {"bound": "host", "achieved": round(value, 1), "peak": None,
                     "unit": "appends/s", "frac": None, "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


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
    ap.add_argument("--graphs", action="store_true",
                    help="capture each step in a HIP graph and replay it (default: launch the "
                         "prepared call directly; for a one-kernel step a graph replay only "
                         "adds a gap between steps)")
    ap.add_argument("--unfused", action="store_true",
                    help="run the step as two calls (reshape_and_cache, then decode)")
    ap.add_argument("--no-groups", action="store_true",
                    help="decode a batch whose sequences share prefix blocks one sequence at "
                         "a time (default: the grouped decode, shared blocks read once per "
                         "group)")
    ap.add_argument("--no-gather", action="store_true",
                    help="skip the gather-ceiling probe that runs after the decode timing")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run copy_blocks on a known byte count (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(no sharding, no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    global torch
    import torch
    import paged_kv_cache_374_amd as pkv
    if args.workload == "block_manager_serving":   # host code: no GPU needed
        bench_block_manager(args)
        return
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    pkv.load()
    if args.workload == "swap_blocks_8b":
        bench_swap(args, pkv, dev)
        return
    if args.workload == "gather_ceiling":
        bench_gather(args, pkv, dev)
        return
    sets = build_sets(args.workload, max(1, args.rotate), dev)
    torch.cuda.synchronize()
    for s in sets:
        prepare(pkv, s, graphs=args.graphs, fused=not args.unfused,
                grouped=not args.no_groups)

    for i in range(args.warmup):
        sets[i % len(sets)].run()
    torch.cuda.synchronize()

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # A batch whose sequences share blocks reads a shared block from HBM once: its value
    # counts the distinct blocks read (the logical bytes are reported beside it).
    shared_sets = all(x.kv_unique < 0.98 * x.kv for x in sets)
    kv_total = kv_logical = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        s = sets[i % len(sets)]
        s.run()
        kv_total += s.kv_unique if shared_sets else s.kv
        kv_logical += s.kv
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = max(start.elapsed_time(stop), 1e-9)
    value = kv_total / (ms * 1e-3) / 1e9
    value_logical = kv_logical / (ms * 1e-3) / 1e9
    s0 = sets[0]
    seqs_per_s = s0.num_seqs * args.steps / (ms * 1e-3)
    # spread of single steps: the same steps again, an event between consecutive steps
    n_spread = max(20, args.steps)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_spread + 1)]
    evs[0].record()
    for i in range(n_spread):
        sets[i % len(sets)].run()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n_spread))
    pct = lambda q: per_step[min(n_spread - 1, int(round(q * (n_spread - 1))))]
    step_spread = {"p10": round(pct(0.1), 3), "p50": round(pct(0.5), 3),
                   "p90": round(pct(0.9), 3), "samples": n_spread,
                   "timing": "one HIP event between consecutive steps, a separate pass after "
                             "the timed steps"}
    # the dominant kernel on its own, back to back over the same pool sets
    dec_us = time_decode_kernel(sets, graphs=args.graphs)
    kv_per_launch = sum(s.kv for s in sets) / len(sets)
    achieved = kv_per_launch / (dec_us * 1e-6) / 1e9
    chunk = s0.query_start is not None
    flops_per_launch = sum(s.flops for s in sets) / len(sets)
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)   # FLOP per byte
    mfma_bound = chunk and flops_per_launch / kv_per_launch > ridge
    tflops = flops_per_launch / (dec_us * 1e-6) / 1e12 if chunk else None

    # blocks shared by several sequences are read once from HBM: price the roofline on
    # the distinct bytes (the logical figure stays in the line as well)
    kv_unique = sum(x.kv_unique for x in sets) / len(sets)
    shared = kv_unique < 0.98 * kv_per_launch
    achieved_hbm = (kv_unique if shared else kv_per_launch) / (dec_us * 1e-6) / 1e9
    gather = None
    if not mfma_bound and not args.no_gather:
        log("[bench] gather ceiling: the probe on the decode's tiles")
        best, sweep = gather_ceiling(pkv, sets)
        gather = {"gbs": best["gbs"], "shape": {k: best[k] for k in ("workgroups",
                                                                       "tiles_in_flight")},
                  "frac": round(achieved / best["gbs"], 4), "sweep": sweep,
                  "what": "pkv_read_tiles on exactly the K and V tiles one decode launch "
                          "reads (whole tiles, non-temporal), best launch shape"}

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline: oracle on the host cores")
        # the last step that used set 0 left its output in set 0's buffer
        if chunk:
            cpu, parity = cpu_baseline_chunk(s0, args.cpu_seconds, mfma_bound)
            cpu.update(cpu_description())
        else:
            one = args.cpu_seconds / 2 if s0.name in ("llama3_8b_decode", "tiny_fp32") else 0
            cpu, parity = cpu_baseline(s0, args.cpu_seconds, one_thread_seconds=one)
            if s0.name == "llama3_8b_decode":
                cpu["tiny_fp32"] = cpu_baseline_tiny()

    if args.calibrate:
        calibrate(pkv, dev)

    grouped_dec = getattr(s0, "groups", None) is not None
    elt = s0.k_cache.element_size()
    dname = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[s0.dtype]
    kv_dname = "fp8_e4m3" if s0.kv_scales is not None else dname
    fp8 = "_fp8" if s0.kv_scales is not None else ""
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
        "value_counts": ("distinct KV blocks read per step (a block shared by several "
                         "sequences once)" if shared_sets else "algorithmic KV bytes per step"),
        "value_logical_gbs": round(value_logical, 2) if shared_sets else None,
        "seqs_per_s": round(seqs_per_s, 1),
        "config": {
            "workload": s0.name,
            "batch": s0.num_seqs,
            "num_heads": s0.num_heads,
            "num_kv_heads": s0.num_kv_heads,
            "head_dim": s0.head_dim,
            "block_size": s0.block_size,
            "num_blocks": s0.num_blocks,
            "kv_dtype": kv_dname,
            "element_bytes": elt,
            "mean_context": round(float(s0.context_lens.float().mean()), 1),
            "kv_bytes_per_step": int(kv_per_launch),
            "kv_unique_block_bytes_per_step": int(sum(x.kv_unique for x in sets) / len(sets)),
            "partition_size": s0.partition_size,
            "pool_sets": len(sets),
            "step": ("reshape_and_cache(chunk tokens) + paged_attention_chunk "
                     f"({s0.max_query_len} query tokens per sequence, causal)" if chunk else
                     ("copy_blocks(K, V) + " if s0.copy_pairs is not None and
                      s0.extra.get("prefix_tokens", 0) % s0.block_size == 0 else "") +
                     (("paged_attention_decode_grouped with the new tokens (each group's "
                       "shared prefix blocks read once per tile of its members, then each "
                       "member's own blocks after its new token is written; one kernel, "
                       "plus a merge kernel for prefixes past 128 blocks)" if s0.fused else
                       "reshape_and_cache(new token) + paged_attention_decode_grouped")
                      if grouped_dec else
                      "paged_attention_decode_append (new token written at each context "
                      "end, then attended; one kernel)" if s0.fused else
                      "reshape_and_cache(new token) + paged_attention_decode")),
            "groups": ({"num_groups": s0.groups.num_groups,
                        "max_group_size": s0.groups.max_group_size,
                        "max_prefix_blocks": s0.groups.max_prefix_blocks}
                       if grouped_dec else None),
            "query_tokens_per_step": int(s0.q.shape[0]),
            "flops_per_step": int(flops_per_launch) if chunk else None,
            "tflops": round(tflops, 2) if chunk else None,
            "launch": "one hip graph per step" if args.graphs else "direct (one call per step)",
            "wall_s_timed": round(wall, 4),
        },
        "step_us": step_spread,
        "roofline": {
            "bound": "mfma" if mfma_bound else "hbm",
            "kernel": ("paged_attention_chunk" if chunk else
                       "paged_attention_decode_grouped" if grouped_dec else
                       "paged_attention_decode_append" if s0.fused
                       else "paged_attention_decode") + fp8,
            "achieved": round(tflops if mfma_bound else achieved_hbm, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS if mfma_bound
                          else achieved_hbm / HBM_PEAK_GBS, 4),
            "bytes": ("distinct blocks read (shared blocks once)" if shared else
                      "algorithmic KV bytes") if not mfma_bound else None,
            "achieved_logical_gbs": round(achieved, 2) if shared else None,
            "traffic": traffic_per_launch(s0.name),
            "launch_us_mean": round(dec_us, 3),
            "launch_timing": "back-to-back decode launches over the pool sets, HIP events",
            "gather_ceiling": gather,
        },
        "cpu_baseline": cpu,
    }
    if parity is not None:
        line["parity_max_abs_err_vs_oracle"] = parity
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
