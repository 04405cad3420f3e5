#!/usr/bin/env python3
"""Benchmark: paged decode on a Llama-3.1-8B-shaped attention layer, one MI355X.

One step = one decode iteration of all 32 layers of the batch: for each layer
(its own K/V block pool, all layers sharing one block table) the new token's
K/V rows are scattered into their slots (kv_cache_write) and the batch's
decode queries attend to every cached token (paged_attn_decode).  32 pools of
~160 MB rotate through HBM, so no layer's KV is still in the 256 MB
Infinity Cache when it is read again.

Printed (one JSON line): effective KV GB/s of the whole step (algorithmic bytes
/ time, inputs resident in HBM), query tokens/s per layer, the live roofline of
the decode call measured with HIP events on the launch stream, and the CPU
oracle timed on a bounded sample on this host's cores.  A step is captured
once in a HIP graph and replayed (the default; --no-graph launches every call
from Python, which on this host is slower than the GPU work it launches).

    python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import concurrent.futures
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode effective KV GB/s (% of HBM peak) and query tokens/s per layer"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    """sha256 over the library's sources and build script: counter-derived
    traffic figures are only reported for the exact code they were taken on."""
    import hashlib
    h = hashlib.sha256()
    files = []
    for d in ("paged_kv_cache_attn_amd/csrc", "include"):
        for name in sorted(os.listdir(os.path.join(ROOT, d))):
            if name.endswith((".hip", ".h")):
                files.append(os.path.join(d, name))
    files.append("paged_kv_cache_attn_amd/build.py")
    for rel in files:
        h.update(rel.encode())
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per call from the FETCH_SIZE / WRITE_SIZE counter runs kept
    under profiles/ (scaled by the copy-kernel calibration), or None when
    they were taken on different sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    e = t.get("workloads", {}).get(workload)
    if not e or t.get("source_sha256") != kernel_source_hash():
        return None
    return e.get("hbm_bytes_per_call")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
# Host threads the oracle may use: every core this process may run on, up to
# the 16 host CPUs the GPU machine allots to one GPU.
HOST_THREAD_CAP = 16


def host_info() -> dict:
    """Core counts and the CPU model of this host (for the CPU-baseline record)."""
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"os_cpu_count": os.cpu_count(), "usable_cores": usable, "cpu_model": model,
            "threads_used": max(1, min(HOST_THREAD_CAP, usable))}
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b_decode",
                    choices=["llama8b_decode", "tiny_decode", "llama8b_decode_f32", "llama70b_long", "llama8b_decode_fp8", "llama70b_long_fp8",
                             "llama70b_one_long",
                             "chunked_prefill_fp8", "shared_prefix", "shared_prefix_cow",
                             "chunked_prefill", "block_size_sweep", "swap", "mixed_decode",
                             "copy_calibration", "llama8b_decode_timeline", "llama70b_long_timeline"])
    ap.add_argument("--layers", type=int, default=0, help="layer pools to rotate (0 = workload default)")
    ap.add_argument("--block-size", type=int, default=16,
                    help="cache block size of the decode and prefill workloads (the headline runs use 16)")
    ap.add_argument("--partition", type=int, default=-1, help="decode partition size (-1 = workload default)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="wall-clock budget of the CPU-oracle sample (seconds, on up to 16 threads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-plan", action="store_true",
                    help="decode without a per-step plan (each call stages its own split)")
    ap.add_argument("--no-fold", action="store_true",
                    help="decode steps as two calls per layer (kv_cache_write, then the planned decode) instead "
                         "of paged_attn_decode_append")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every call from Python instead of replaying captured HIP graphs")
    return ap.parse_args()


STEP_STATS = {}  # per-step time distribution (ms) of the last graph-timed run
GRAPHS = {}      # the last graph-timed run's step graph (for the cold-layer measurement)


def time_calls(args, torch, layers, call):
    """Mean ms of call(l) over the layers, timed like the attention calls
    (a replayed graph of the `layers` calls, or eager events)."""
    if args.no_graph:
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            for l in range(layers):
                call(l)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / (args.steps * layers)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for l in range(layers):
            call(l)
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / (args.steps * layers)


def measured_copy_gbs(torch):
    """Read + write GB/s of a 1 GiB device-to-device copy on this GPU (the
    practical bandwidth a streaming kernel can be compared with)."""
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(10):
        y.copy_(x)
    t1.record()
    torch.cuda.synchronize()
    gbs = 2 * n * 10 / (t0.elapsed_time(t1) * 1e-3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    return round(gbs, 1)


def time_layers(args, torch, layers, write, call, out, pre=None):
    """Time one step (every layer: write(l) then call(l)) and the attention call alone.

    Default: each is captured once in a HIP graph (a decode step is a fixed
    sequence of launches, replayed every token) and the graphs are replayed
    between two events on the launch stream; per-call time is the replay time
    of a graph holding the `layers` attention calls alone, divided by
    `layers`.  Before timing, a replay of the step graph must reproduce the
    eager result of the last layer bit for bit.  With --no-graph every call is
    launched from Python and bracketed by pre-created event pairs.
    `pre` (optional) runs once at the start of a step and of the call-only
    graph (a decode plan shared by the step's layers); its time is included.
    Returns (ms per step, ms per call, wall seconds of the timed steps, mode).
    """
    def step():
        if pre is not None:
            pre()
        for l in range(layers):
            write(l)
            call(l)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.no_graph:
        n = args.steps * layers
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        wall0 = time.perf_counter()
        t0.record()
        i = 0
        for _ in range(args.steps):
            if pre is not None:
                pre()
            for l in range(layers):
                write(l)
                ev[i][0].record()
                call(l)
                ev[i][1].record()
                i += 1
        t1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        return (t0.elapsed_time(t1) / args.steps, float(np.mean([a.elapsed_time(b) for a, b in ev])), wall,
                "eager")
    g_step, g_call = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_step):
        step()
    GRAPHS["step"] = g_step
    with torch.cuda.graph(g_call):
        if pre is not None:
            pre()
        for l in range(layers):
            call(l)
    g_step.replay()
    torch.cuda.synchronize()
    replayed = out.clone()
    write(layers - 1)
    call(layers - 1)
    torch.cuda.synchronize()
    if not torch.equal(replayed, out):
        raise SystemExit("bench.py: graph replay differs from the eager call")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    wall0 = time.perf_counter()
    ev[0].record()
    for i in range(args.steps):
        g_step.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    STEP_STATS.update(p10=round(float(np.percentile(per, 10)), 4), p50=round(float(np.median(per)), 4),
                      p90=round(float(np.percentile(per, 90)), 4))
    ms_step = ev[0].elapsed_time(ev[-1]) / args.steps
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        g_call.replay()
    t1.record()
    torch.cuda.synchronize()
    ms_call = t0.elapsed_time(t1) / (args.steps * layers)
    return ms_step, ms_call, wall, "hip-graph"


def cold_layer_ms(torch, step_graph_replay, one_layer, reps=5):
    """Median GPU time of one layer's attention (its plan included) replayed right after a whole step,
    so that layer's K/V has been pushed out of the caches by the other layers' streams."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one_layer()
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        step_graph_replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return float(np.median(times))


def cpu_oracle_decode(q, k, v, tables, lens, scale, budget_s, kv_scales=(None, None), threads=None):
    """Time the oracle over whole passes of the batch (all sequences, one layer) on `threads` host threads
    (default: every usable core up to HOST_THREAD_CAP); the first pass's output is returned for parity."""
    import oracle
    oracle.build(force=False)
    cores = threads or host_info()["threads_used"]
    B = q.shape[0]

    def one(b):
        return oracle.paged_decode(q[b:b + 1], k, v, tables[b:b + 1], lens[b:b + 1], scale,
                                   k_scale=kv_scales[0], v_scale=kv_scales[1])

    outs = None
    passes = 0
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(max_workers=cores) as ex:
        # order longest first so the pool stays busy
        order = list(np.argsort(-lens))
        while True:
            res = dict(zip(order, ex.map(one, order)))
            passes += 1
            if outs is None:
                outs = np.concatenate([res[b] for b in range(B)])
            if time.perf_counter() - t0 >= budget_s:
                break
    return outs, passes, time.perf_counter() - t0, cores


def fp8_pool(torch, W, shape, std, seed):
    """An FP8 E4M3 layer pool: N(0, std) values quantised with the per-tensor scale
    max|x| / 448 (torch's float8 conversion; input preparation only)."""
    x = W.device_values(shape, std, seed, "f32")
    s = float(x.abs().max()) / 448.0
    codes = (x / s).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    del x
    return codes, s


def bench_decode(args, torch, pa, W, w, layers, partition, fp8=False):
    dev = "cuda"
    B, Hq, Hkv, D = w.layout.batch, w.num_heads, w.num_kv_heads, w.head_dim
    lens = w.layout.seq_lens
    max_len = int(lens.max())
    shape = w.cache_shape()
    # per-layer pools, drawn on the device
    if fp8:
        KS = [fp8_pool(torch, W, shape, w.std, w.seed * 1000 + 2 * l) for l in range(layers)]
        VS = [fp8_pool(torch, W, shape, w.std, w.seed * 1000 + 2 * l + 1) for l in range(layers)]
        K, ks = [a for a, _ in KS], [s for _, s in KS]
        V, vs = [a for a, _ in VS], [s for _, s in VS]
    else:
        K = [W.device_values(shape, w.std, w.seed * 1000 + 2 * l, w.dtype) for l in range(layers)]
        V = [W.device_values(shape, w.std, w.seed * 1000 + 2 * l + 1, w.dtype) for l in range(layers)]
    q = W.device_values((B, Hq, D), w.std, w.seed * 1000 - 1, w.dtype)
    newk = W.device_values((B, Hkv, D), w.std, w.seed * 1000 - 2, w.dtype)
    newv = W.device_values((B, Hkv, D), w.std, w.seed * 1000 - 3, w.dtype)
    slots = torch.from_numpy(np.array([w.layout.block_tables[b, (lens[b] - 1) // w.block_size] * w.block_size
                                       + (lens[b] - 1) % w.block_size for b in range(B)], np.int64)).to(dev)
    bt = torch.from_numpy(w.layout.block_tables).to(dev)
    sl = torch.from_numpy(lens.astype(np.int32)).to(dev)
    out = torch.empty(B, Hq, D, device=dev, dtype=torch.float32)
    wsb = pa.paged_attn_decode_workspace_size(B, Hq, Hkv, D, w.block_size, max_len, partition)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    scale = w.scale

    # one plan per step serves all layers (same block tables and lengths)
    kvd = pa.PA_FP8_E4M3 if fp8 else pa._dtype_code(K[0])
    psize = pa.paged_attn_decode_plan_size(B, Hq, Hkv, D, w.block_size, w.layout.block_tables.shape[1], max_len,
                                           partition, kvd)
    use_plan = not args.no_plan and psize > 0
    plan = torch.empty(max(psize, 1), dtype=torch.uint8, device=dev) if use_plan else None
    pre = (lambda: pa.paged_attn_decode_plan(plan, K[0], bt, sl, Hq, max_len, partition)) if use_plan else None
    if fp8:
        write = lambda l: pa.kv_cache_write_fp8(newk, newv, K[l], V[l], slots, ks[l], vs[l])
    else:
        write = lambda l: pa.kv_cache_write(newk, newv, K[l], V[l], slots)
    # the step's write folded into the attention call (the balanced bf16 path)
    fold = use_plan and not fp8 and w.dtype == "bf16" and not args.no_fold
    if fold:
        write = lambda l: None
        call = lambda l: pa.paged_attn_decode_append(out, q, newk, newv, slots, K[l], V[l], plan, bt, sl, scale,
                                                     max_len, partition, ws)
    elif use_plan:
        call = lambda l: pa.paged_attn_decode_planned(out, q, K[l], V[l], plan, bt, sl, scale, max_len, partition,
                                                      ws, k_scale=ks[l] if fp8 else 1.0,
                                                      v_scale=vs[l] if fp8 else 1.0)
    elif fp8:
        call = lambda l: pa.paged_attn_decode_fp8(out, q, K[l], V[l], ks[l], vs[l], bt, sl, scale, max_len,
                                                  partition, ws)
    else:
        call = lambda l: pa.paged_attn_decode(out, q, K[l], V[l], bt, sl, scale, max_len, partition, ws)
    ms_step, ms_decode, wall, mode = time_layers(args, torch, layers, write, call, out, pre)
    copy_gbs = measured_copy_gbs(torch)
    if fp8:
        # 1-byte K/V rows, bf16 q, fp32 out, table entries, lengths
        nblk = (lens.astype(np.int64) + w.block_size - 1) // w.block_size
        dec_bytes = int(lens.astype(np.int64).sum()) * Hkv * D * 2 + B * Hq * D * (2 + 4) + 4 * int(nblk.sum()) + 4 * B
        write_bytes = B * Hkv * D * (2 + 1) * 2 + 8 * B
    else:
        dec_bytes = w.algorithmic_bytes(out_bytes=4)
        write_bytes = B * Hkv * D * w.elem_bytes * 2 * 2 + 8 * B
    step_bytes = layers * (dec_bytes + write_bytes)
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    call_bytes = dec_bytes + (write_bytes if fold else 0)  # a folded call also moves the new rows
    achieved = call_bytes / (ms_decode * 1e-3) / 1e9

    # one layer's attention (plan included) with its K/V cold: replayed right after a whole step
    cold_ms = None
    if mode == "hip-graph":
        def one_layer():
            if pre is not None:
                pre()
            call(0)
        cold_ms = cold_layer_ms(torch, GRAPHS["step"].replay, one_layer)

    # parity on the first and the last layer of the rotation, and the CPU baseline on layer 0 (the
    # oracle on the host copies): all usable cores, then one core
    def gpu_layer(l):
        torch.cuda.synchronize()
        if pre is not None:
            pre()
        call(l)
        torch.cuda.synchronize()
        return out.double().cpu().numpy()

    def host(t):
        t = t.contiguous().cpu()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    cpu = None
    parity = None
    parity_last = None
    if not args.no_cpu_baseline:
        hi = host_info()
        gpu_out = gpu_layer(0)
        hq = host(q)
        ref, passes, secs, cores = cpu_oracle_decode(hq, host(K[0]), host(V[0]), w.layout.block_tables,
                                                     lens, scale, 0.6 * args.cpu_seconds,
                                                     (ks[0], vs[0]) if fp8 else (None, None))
        parity = float(np.max(np.abs(gpu_out - ref)))
        _, passes1, secs1, _ = cpu_oracle_decode(hq, host(K[0]), host(V[0]), w.layout.block_tables, lens, scale,
                                                 0.4 * args.cpu_seconds, (ks[0], vs[0]) if fp8 else (None, None),
                                                 threads=1)
        gpu_last = gpu_layer(layers - 1)
        ref_last, _, _, _ = cpu_oracle_decode(hq, host(K[layers - 1]), host(V[layers - 1]), w.layout.block_tables,
                                              lens, scale, 0.0,
                                              (ks[layers - 1], vs[layers - 1]) if fp8 else (None, None))
        parity_last = float(np.max(np.abs(gpu_last - ref_last)))
        cpu = {"value": round(passes * dec_bytes / secs / 1e9, 4), "unit": "GB/s", "cores": cores,
               "kind": "oracle",
               "sample": "%d full pass(es) of layer 0 (%d sequences, %d tokens) through the fp64 C oracle, "
                         "%.1f s, sequences spread over %d threads" % (passes, B, int(lens.sum()), secs, cores),
               "one_core": {"value": round(passes1 * dec_bytes / secs1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                            "sample": "%d full pass(es) of layer 0 on one thread, %.1f s" % (passes1, secs1)},
               "query_tokens_per_s": round(passes * B / secs, 1),
               "host": hi}
    res = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3 KV, bf16 q" if fp8 else w.dtype, "data": "synthetic",
        "config": {"workload": (w.name.replace("_bf16", "_fp8") if fp8 else w.name), "batch": B, "num_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": D,
                   "block_size": w.block_size, "layers": layers, "total_tokens": int(lens.sum()),
                   "max_seq_len": max_len, "partition_size": partition or "auto",
                   "num_blocks_per_layer": w.layout.num_blocks},
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "query_tokens_per_s_per_layer": round(B / (ms_step * 1e-3 / layers), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic((w.name.replace("_bf16", "_fp8") if fp8 else w.name)),
                     "traffic_unit": "bytes per call",
                     "kernel": ("paged_attn_decode_fp8 call" if fp8 else
                                "paged_attn_decode_append call (write folded in)" if fold else "paged_attn_decode call"),
                     "bytes_per_launch": call_bytes,
                     "avg_launch_ms": round(ms_decode, 5)},
        "cpu_baseline": cpu,
        "parity_max_abs_err_layer0": parity,
        "parity_max_abs_err_last_layer": parity_last,
        "cold_layer_us": None if cold_ms is None else round(cold_ms * 1e3, 2),
        "timing": mode, "ms_per_step_p10_p50_p90": [STEP_STATS.get(k) for k in ("p10", "p50", "p90")],
        "copy_GBs_read_plus_write": copy_gbs, "wall_s": round(wall, 3),
        "decode_plan": "one plan per step, shared by the layers" if use_plan else None,
        "step_calls_per_layer": ("paged_attn_decode_append (the new token's K/V write folded into the attention "
                                 "kernels)" if fold else "kv_cache_write, then the decode"),
    }
    return res


def bench_decode_timeline(args, torch, pa, W, w, layers):
    """Phases of one folded decode call (plan once per step, then paged_attn_decode_append per layer) from
    the timestamp build: each workgroup of the main and merge kernels records the s_memrealtime clock
    (100 MHz) at fixed points (include/paged_attn.h, pa_timeline).  The step is captured as a HIP graph
    and replayed; after each replay the stamps hold the step's last call, which ran right after the one
    before it.  Each XCD has its own clock, so stamps are only compared within an XCD; workgroup id i is
    taken to run on XCD i mod 8 (the dispatch's round robin), which the start spread on each XCD checks."""
    dev = "cuda"
    B, Hq, Hkv, D = w.layout.batch, w.num_heads, w.num_kv_heads, w.head_dim
    lens = w.layout.seq_lens
    max_len = int(lens.max())
    tlib = pa.load_timeline_library()
    with pa.using_library(tlib):
        K = [W.device_values(w.cache_shape(), w.std, w.seed * 1000 + 2 * l, w.dtype) for l in range(layers)]
        V = [W.device_values(w.cache_shape(), w.std, w.seed * 1000 + 2 * l + 1, w.dtype) for l in range(layers)]
        q = W.device_values((B, Hq, D), w.std, w.seed * 1000 - 1, w.dtype)
        newk = W.device_values((B, Hkv, D), w.std, w.seed * 1000 - 2, w.dtype)
        newv = W.device_values((B, Hkv, D), w.std, w.seed * 1000 - 3, w.dtype)
        slots = torch.from_numpy(np.array([w.layout.block_tables[b, (lens[b] - 1) // w.block_size] * w.block_size
                                           + (lens[b] - 1) % w.block_size for b in range(B)], np.int64)).to(dev)
        bt = torch.from_numpy(w.layout.block_tables).to(dev)
        sl = torch.from_numpy(lens.astype(np.int32)).to(dev)
        out = torch.empty(B, Hq, D, device=dev, dtype=torch.float32)
        ws = torch.empty(max(pa.paged_attn_decode_workspace_size(B, Hq, Hkv, D, w.block_size, max_len, 0), 1),
                         dtype=torch.uint8, device=dev)
        psize = pa.paged_attn_decode_plan_size(B, Hq, Hkv, D, w.block_size, w.layout.block_tables.shape[1],
                                               max_len, 0, pa.PA_BF16)
        plan = torch.empty(max(psize, 1), dtype=torch.uint8, device=dev)

        def step():
            pa.paged_attn_decode_plan(plan, K[0], bt, sl, Hq, max_len, 0)
            for l in range(layers):
                pa.paged_attn_decode_append(out, q, newk, newv, slots, K[l], V[l], plan, bt, sl, w.scale,
                                            max_len, 0, ws)

        for _ in range(max(args.warmup, 1)):
            step()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        pa.timeline(tlib, pa.PA_TIMELINE_ROWS, clear=True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms_step = e0.elapsed_time(e1) / args.steps
        reps = []
        for _ in range(args.steps):
            g.replay()
            reps.append(pa.timeline(tlib, pa.PA_TIMELINE_ROWS, clear=True))

    def pct(a, q):
        return float(np.percentile(a, q)) if len(a) else None

    per = []
    for main, merge in reps:
        m = main.astype(np.int64)
        g_ = merge.astype(np.int64)
        ids = np.nonzero(m[:, 0] > 0)[0]
        mids = np.nonzero(g_[:, 0] > 0)[0]
        mm = m[ids] / 100.0  # us
        waves = mm[:, 2:6]
        r = {"workgroups": int(len(ids)), "merge_workgroups": int(len(mids)),
             "prologue": mm[:, 1] - mm[:, 0], "stream": (waves - mm[:, 1:2]).ravel(),
             "wave_spread": waves.max(1) - waves.min(1), "barrier": mm[:, 6] - waves.max(1),
             "combine": mm[:, 7] - mm[:, 6], "workgroup": mm[:, 7] - mm[:, 0],
             "merge": (g_[mids, 1] - g_[mids, 0]) / 100.0}
        xs = {k: [] for k in ("start_spread", "main_span", "tail", "boundary", "merge_span", "call")}
        for x in range(8):
            ix = ids[ids % 8 == x]
            gx = mids[mids % 8 == x]
            if not len(ix) or not len(gx):
                continue
            st, en = m[ix, 0] / 100.0, m[ix, 7] / 100.0
            ms_, me_ = g_[gx, 0] / 100.0, g_[gx, 1] / 100.0
            xs["start_spread"].append(st.max() - st.min())
            xs["main_span"].append(en.max() - st.min())
            xs["tail"].append(en.max() - np.median(en))
            xs["boundary"].append(ms_.min() - en.max())
            xs["merge_span"].append(me_.max() - ms_.min())
            xs["call"].append(me_.max() - st.min())
        r.update({k: np.array(v) for k, v in xs.items()})
        per.append(r)

    def summary(key, qs=(5, 50, 95)):
        # per call: the percentiles over its workgroups (or XCDs); then the median over calls
        vals = [[pct(r[key], q_) for q_ in qs] for r in per if len(r[key])]
        return [round(float(np.median([v[i] for v in vals])), 2) for i in range(len(qs))] if vals else None

    phases = {
        "main_start_spread_per_xcd_us_p5_p50_p95": summary("start_spread"),
        "prologue_us_p5_p50_p95": summary("prologue"),
        "stream_per_wave_us_p5_p50_p95": summary("stream"),
        "wave_end_spread_in_workgroup_us_p5_p50_p95": summary("wave_spread"),
        "barrier_after_last_wave_us_p5_p50_p95": summary("barrier"),
        "combine_us_p5_p50_p95": summary("combine"),
        "workgroup_start_to_end_us_p5_p50_p95": summary("workgroup"),
        "main_kernel_span_per_xcd_us_p5_p50_p95": summary("main_span"),
        "main_tail_after_median_workgroup_end_per_xcd_us_p5_p50_p95": summary("tail"),
        "boundary_main_end_to_merge_start_per_xcd_us_p5_p50_p95": summary("boundary"),
        "merge_workgroup_us_p5_p50_p95": summary("merge"),
        "merge_span_per_xcd_us_p5_p50_p95": summary("merge_span"),
        "call_span_per_xcd_us_p5_p50_p95": summary("call"),
    }
    call = phases["call_span_per_xcd_us_p5_p50_p95"]
    spread = phases["main_start_spread_per_xcd_us_p5_p50_p95"]
    return {
        "metric": "phases of one paged_attn_decode_append call (timestamp build, per-workgroup clocks)",
        "value": call[1] if call else None, "unit": "us (median over XCDs of main start to merge end)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name + "_timeline", "batch": B, "num_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": D, "block_size": w.block_size, "layers": layers, "total_tokens": int(lens.sum())},
        "workgroups": per[0]["workgroups"] if per else 0, "merge_workgroups": per[0]["merge_workgroups"] if per else 0,
        "calls_sampled": len(per), "phases": phases,
        "xcd_round_robin_consistent": bool(spread is not None and spread[2] < 5.0),
        "graph_us_per_call_timestamp_build": round(ms_step * 1e3 / layers, 2),
    }


def host_copy(torch, t):
    t = t.contiguous().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def bench_prefill(args, torch, pa, W, w, layers, fp8=False):
    """Chunked prefill: per layer, write the chunk's K/V rows, then causal chunk attention."""
    dev = "cuda"
    B, Hq, Hkv, D = w.layout.batch, w.num_heads, w.num_kv_heads, w.head_dim
    Tq = w.num_query_tokens
    shape = (w.layout.num_blocks, Hkv, w.layout.block_size, D)
    if fp8:
        KS = [fp8_pool(torch, W, shape, w.std, w.seed * 1000 + 2 * l) for l in range(layers)]
        VS = [fp8_pool(torch, W, shape, w.std, w.seed * 1000 + 2 * l + 1) for l in range(layers)]
        K, ks = [a for a, _ in KS], [s for _, s in KS]
        V, vs = [a for a, _ in VS], [s for _, s in VS]
    else:
        K = [W.device_values(shape, w.std, w.seed * 1000 + 2 * l, w.dtype) for l in range(layers)]
        V = [W.device_values(shape, w.std, w.seed * 1000 + 2 * l + 1, w.dtype) for l in range(layers)]
    q = W.device_values((Tq, Hq, D), w.std, w.seed * 1000 - 1, w.dtype)
    newk = W.device_values((Tq, Hkv, D), w.std, w.seed * 1000 - 2, w.dtype)
    newv = W.device_values((Tq, Hkv, D), w.std, w.seed * 1000 - 3, w.dtype)
    slots = torch.from_numpy(w.chunk_slots()).to(dev)
    bt = torch.from_numpy(w.layout.block_tables).to(dev)
    sl = torch.from_numpy(w.layout.seq_lens.astype(np.int32)).to(dev)
    qsl = torch.from_numpy(w.query_start_loc).to(dev)
    out = torch.empty(Tq, Hq, D, device=dev, dtype=torch.float32)
    max_q, max_len = int(w.chunk_lens.max()), int(w.layout.seq_lens.max())

    if fp8:
        write = lambda l: pa.kv_cache_write_fp8(newk, newv, K[l], V[l], slots, ks[l], vs[l])
        call = lambda l: pa.paged_attn_prefill_chunk_fp8(out, q, K[l], V[l], ks[l], vs[l], bt, qsl, sl, w.scale,
                                                         max_q, max_len)
        write_bytes = Tq * Hkv * D * (2 + 1) * 2 + 8 * Tq  # bf16 rows read, codes written, + slots
    else:
        write = lambda l: pa.kv_cache_write(newk, newv, K[l], V[l], slots)
        call = lambda l: pa.paged_attn_prefill_chunk(out, q, K[l], V[l], bt, qsl, sl, w.scale, max_q, max_len)
        write_bytes = Tq * Hkv * D * 2 * 2 * 2 + 8 * Tq  # K and V rows read and written, bf16, + slots
    ms_step, ms_call, wall, mode = time_layers(args, torch, layers, write, call, out)
    ms_write = time_calls(args, torch, layers, write)
    flops = w.flops()
    tflops = flops / (ms_call * 1e-3) / 1e12
    # sampled parity: the last 8 rows of sequence 0 and the first 8 rows of the last sequence,
    # each checked as a chunk of its own (a chunk's rows depend only on their positions)
    call(0)
    torch.cuda.synchronize()
    import oracle
    kvs = dict(k_scale=ks[0], v_scale=vs[0]) if fp8 else {}
    oracle.build(force=False)
    hq, hk, hv = host_copy(torch, q), host_copy(torch, K[0]), host_copy(torch, V[0])
    qsl_h = w.query_start_loc
    errs = []
    for b, (i0, i1) in ((0, (504, 512)), (B - 1, (0, 8))):
        S, n = int(w.layout.seq_lens[b]), int(w.chunk_lens[b])
        rows = slice(qsl_h[b] + i0, qsl_h[b] + i1)
        ref = oracle.paged_prefill(hq[rows], hk, hv, w.layout.block_tables[b:b + 1], np.array([0, i1 - i0], np.int32),
                                   np.array([S - n + i1], np.int32), w.scale, **kvs)
        errs.append(float(np.max(np.abs(out[rows].double().cpu().numpy() - ref))))
    cpu = None
    if not args.no_cpu_baseline:
        hi = host_info()
        b = 0
        S, n = int(w.layout.seq_lens[b]), int(w.chunk_lens[b])

        def one(i):
            r_ = slice(qsl_h[b] + i, qsl_h[b] + i + 1)
            return oracle.paged_prefill(hq[r_], hk, hv, w.layout.block_tables[b:b + 1], np.array([0, 1], np.int32),
                                        np.array([S - n + i + 1], np.int32), w.scale, **kvs)

        def timed_rows(threads, budget):
            """Chunk rows of sequence 0 (all query heads) through the oracle on `threads` threads, in
            batches, until the budget is spent; returns (rows, seconds, TFLOP/s)."""
            t0 = time.perf_counter()
            rows_done = 0
            step = 4 * threads
            with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
                i = 0
                while time.perf_counter() - t0 < budget and i < n:
                    list(ex.map(one, range(i, min(i + step, n))))
                    rows_done += min(step, n - i)
                    i += step
            secs = time.perf_counter() - t0
            keys = sum((S - n + i + 1) for i in range(rows_done))
            return rows_done, secs, 4.0 * keys * Hq * D / secs / 1e12

        cores = hi["threads_used"]
        rows_done, secs, tf = timed_rows(cores, 0.6 * args.cpu_seconds)
        rows1, secs1, tf1 = timed_rows(1, 0.4 * args.cpu_seconds)
        cpu = {"value": round(tf, 6), "unit": "TFLOP/s", "cores": cores,
               "kind": "oracle",
               "sample": "%d chunk rows of sequence 0 (all %d query heads) through the fp64 C oracle, %.1f s, "
                         "rows spread over %d threads" % (rows_done, Hq, secs, cores),
               "one_core": {"value": round(tf1, 6), "unit": "TFLOP/s", "cores": 1,
                            "sample": "%d chunk rows of sequence 0 on one thread, %.1f s" % (rows1, secs1)},
               "host": hi}
    return {
        "metric": "chunked prefill attention TFLOP/s and query tokens/s per layer", "value": round(tflops, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 KV, bf16 q" if fp8 else w.dtype, "data": "synthetic",
        "config": {"workload": (w.name.replace("_bf16", "_fp8") if fp8 else w.name), "batch": B,
                   "prefix": int(w.layout.seq_lens[0] - w.chunk_lens[0]),
                   "chunk": int(w.chunk_lens[0]), "num_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
                   "block_size": w.layout.block_size, "layers": layers},
        "query_tokens_per_s_per_layer": round(Tq / (ms_call * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic((w.name.replace("_bf16", "_fp8") if fp8 else w.name)), "traffic_unit": "bytes per call",
                     "kernel": "paged_attn_prefill_chunk%s call" % ("_fp8" if fp8 else ""), "flops_per_launch": flops,
                     "avg_launch_ms": round(ms_call, 5)},
        "kv_cache_write": {"rows": Tq * Hkv, "us_per_call": round(ms_write * 1e3, 3),
                           "GBs": round(write_bytes / (ms_write * 1e-3) / 1e9, 1)},
        "cpu_baseline": cpu, "parity_max_abs_err_sampled_rows": max(errs), "timing": mode,
        "ms_per_step_p10_p50_p90": [STEP_STATS.get(k) for k in ("p10", "p50", "p90")],
        "wall_s": round(wall, 3),
    }


def bench_shared_prefix(args, torch, pa, W, w, layers):
    """Parallel sampling over shared prompt blocks: new-token write + decode; CoW block copies timed apart."""
    dev = "cuda"
    B, Hq, Hkv, D = w.layout.batch, w.num_heads, w.num_kv_heads, w.head_dim
    lens = w.layout.seq_lens
    max_len = int(lens.max())
    shape = w.cache_shape()
    K = [W.device_values(shape, w.std, w.seed * 1000 + 2 * l, w.dtype) for l in range(layers)]
    V = [W.device_values(shape, w.std, w.seed * 1000 + 2 * l + 1, w.dtype) for l in range(layers)]
    q = W.device_values((B, Hq, D), w.std, w.seed * 1000 - 1, w.dtype)
    newk = W.device_values((B, Hkv, D), w.std, w.seed * 1000 - 2, w.dtype)
    newv = W.device_values((B, Hkv, D), w.std, w.seed * 1000 - 3, w.dtype)
    slots = torch.from_numpy(np.asarray(w.extra["new_slots"], np.int64)).to(dev)
    bt = torch.from_numpy(w.layout.block_tables).to(dev)
    sl = torch.from_numpy(lens.astype(np.int32)).to(dev)
    out = torch.empty(B, Hq, D, device=dev, dtype=torch.float32)
    wsb = pa.paged_attn_decode_workspace_size(B, Hq, Hkv, D, w.block_size, max_len, 0)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    copies = w.copies
    pairs = torch.from_numpy(np.asarray(copies, np.int64).reshape(-1, 2)).to(dev)

    psize = pa.paged_attn_decode_plan_size(B, Hq, Hkv, D, w.block_size, w.layout.block_tables.shape[1], max_len, 0,
                                           pa.PA_BF16)
    use_plan = not args.no_plan and psize > 0
    plan = torch.empty(max(psize, 1), dtype=torch.uint8, device=dev) if use_plan else None
    pre = (lambda: pa.paged_attn_decode_plan(plan, K[0], bt, sl, Hq, max_len, 0)) if use_plan else None
    if use_plan:
        call = lambda l: pa.paged_attn_decode_planned(out, q, K[l], V[l], plan, bt, sl, w.scale, max_len, 0, ws)
    else:
        call = lambda l: pa.paged_attn_decode(out, q, K[l], V[l], bt, sl, w.scale, max_len, 0, ws)
    ms_step, ms_call, wall, mode = time_layers(
        args, torch, layers, lambda l: pa.kv_cache_write(newk, newv, K[l], V[l], slots), call, out, pre)
    logical = w.algorithmic_bytes(out_bytes=4)
    unique = w.extra["unique_blocks"] * w.block_size * Hkv * D * w.elem_bytes * 2
    copy = None
    if len(copies):
        # the layers' copies in one HIP graph, replayed (a Python launch loop
        # would time the host, not the copies)
        for _ in range(3):
            pa.block_copy(K[0], V[0], pairs)
        torch.cuda.synchronize()
        gcp = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gcp):
            for l in range(layers):
                pa.block_copy(K[l], V[l], pairs)
        gcp.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            gcp.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (layers * args.steps)
        cbytes = len(copies) * 2 * 2 * Hkv * w.block_size * D * w.elem_bytes  # K and V, read + write
        copy = {"pairs": len(copies), "us_per_call": round(us, 3), "GBs": round(cbytes / us / 1e3, 1)}
    if pre is not None:
        pre()
    call(0)
    torch.cuda.synchronize()
    import oracle
    oracle.build(force=False)
    sel = np.arange(0, B, max(1, B // 16))
    ref = oracle.paged_decode(host_copy(torch, q)[sel], host_copy(torch, K[0]), host_copy(torch, V[0]),
                              w.layout.block_tables[sel], lens[sel], w.scale)
    err = float(np.max(np.abs(out.double().cpu().numpy()[sel] - ref)))
    gbs = logical / (ms_call * 1e-3) / 1e9
    return {
        "metric": METRIC, "value": round(layers * (logical + B * Hkv * D * w.elem_bytes * 4 + 8 * B)
                                         / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "prompts": w.extra["prompts"], "samples": w.extra["samples"],
                   "prompt_len": w.extra["prompt_len"], "layers": layers, "total_tokens": int(lens.sum()),
                   "unique_blocks": w.extra["unique_blocks"], "cow_pairs": len(copies)},
        "query_tokens_per_s_per_layer": round(B / (ms_step * 1e-3 / layers), 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(w.name),
                     "traffic_unit": "bytes per call", "kernel": "paged_attn_decode call (logical KV bytes)", "bytes_per_launch": logical,
                     "unique_kv_bytes": unique, "unique_GBs": round(unique / (ms_call * 1e-3) / 1e9, 2),
                     "avg_launch_ms": round(ms_call, 5)},
        "block_copy": copy, "cpu_baseline": None, "parity_max_abs_err_sampled": err, "timing": mode,
        "decode_plan": "one plan per step, shared by the layers" if use_plan else None,
        "ms_per_step_p10_p50_p90": [STEP_STATS.get(k) for k in ("p10", "p50", "p90")], "wall_s": round(wall, 3),
    }


def slot_waste(layout):
    """Internal fragmentation of a layout: the unused slots of every sequence's last block."""
    lens = layout.seq_lens.astype(np.int64)
    alloc = int((((lens + layout.block_size - 1) // layout.block_size) * layout.block_size).sum())
    return alloc - int(lens.sum()), alloc


def bench_block_sizes(args, torch, pa, W):
    """The 8B decode batch and the chunked prefill at block sizes 8 ... 128: kernel
    time, effective bandwidth / MFMA rate, and the slots the block size wastes
    (the unused tail of each sequence's last block)."""
    import copy as _copy
    sub = _copy.copy(args)
    sub.no_cpu_baseline = True
    rows = []
    for bs in (8, 16, 32, 64, 128):
        w = W.llama8b_decode(block_size=bs)
        d = bench_decode(sub, torch, pa, W, w, args.layers or 32, 0)
        p_w = W.chunked_prefill(block_size=bs)
        p = bench_prefill(sub, torch, pa, W, p_w, args.layers or 32)
        waste, alloc = slot_waste(w.layout)
        rows.append({
            "block_size": bs,
            "decode_us_per_call": round(d["roofline"]["avg_launch_ms"] * 1e3, 3),
            "decode_kernel_GBs": d["roofline"]["achieved"], "decode_step_GBs": d["value"],
            "decode_ms_per_step_p50": d["ms_per_step_p10_p50_p90"][1],
            "prefill_us_per_call": round(p["roofline"]["avg_launch_ms"] * 1e3, 3),
            "prefill_TFLOPs": p["roofline"]["achieved"],
            "decode_slots_allocated": alloc, "decode_slots_wasted": waste,
            "waste_frac": round(waste / alloc, 4), "table_entries": int(alloc // bs),
            "prefill_parity_max_abs_err_sampled_rows": p["parity_max_abs_err_sampled_rows"],
        })
        print("block size %d: decode %.1f us, prefill %.1f us, waste %.2f%%" % (
            bs, rows[-1]["decode_us_per_call"], rows[-1]["prefill_us_per_call"], 100 * rows[-1]["waste_frac"]),
            file=sys.stderr, flush=True)
        del d, p
        torch.cuda.empty_cache()
    ref = next(r for r in rows if r["block_size"] == 16)
    return {
        "metric": METRIC, "value": ref["decode_step_GBs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ref["decode_ms_per_step_p50"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "block_size_sweep", "decode": "llama8b_decode_bf16 lengths at each block size",
                   "prefill": "chunked_prefill_bf16 at each block size", "layers": args.layers or 32,
                   "value_is": "decode step GB/s at block size 16"},
        "sweep": rows, "cpu_baseline": None,
    }


def bench_mixed_decode(args, torch, pa, W):
    """32 decode steps of one batch mixing beam search (16 groups x 4 beams), parallel sampling
    (8 groups x 4 samples) and 32 greedy rows, 32 layers: per step and layer, the step's
    copy-on-write block copies (one block_copy), the new tokens' K/V (kv_cache_write), then
    decode attention through that step's block tables.  The whole trace is captured in one HIP
    graph and replayed; layer 0 of an eager pass is checked against the oracle replaying the
    same copies and writes on the host."""
    import oracle
    dev = "cuda"
    tr = W.mixed_decode_trace()
    layers = args.layers or 32
    B, Hq, Hkv, D, bs = tr.batch, tr.num_heads, tr.num_kv_heads, tr.head_dim, tr.block_size
    shape = (tr.num_blocks, Hkv, bs, D)
    K = [W.device_values(shape, tr.std, tr.seed * 1000 + 2 * l, tr.dtype) for l in range(layers)]
    V = [W.device_values(shape, tr.std, tr.seed * 1000 + 2 * l + 1, tr.dtype) for l in range(layers)]
    k0, v0 = host_copy(torch, K[0]), host_copy(torch, V[0])
    q = W.device_values((B, Hq, D), tr.std, tr.seed * 1000 - 1, tr.dtype)
    newk = W.device_values((B, Hkv, D), tr.std, tr.seed * 1000 - 2, tr.dtype)
    newv = W.device_values((B, Hkv, D), tr.std, tr.seed * 1000 - 3, tr.dtype)
    S = len(tr.tables)
    bt = [torch.from_numpy(t).to(dev) for t in tr.tables]
    sl = [torch.from_numpy(x).to(dev) for x in tr.seq_lens]
    slots = [torch.from_numpy(x).to(dev) for x in tr.slots]
    pairs = [torch.from_numpy(np.asarray(c, np.int64).reshape(-1, 2)).to(dev) for c in tr.copies]
    max_len = int(max(int(x.max()) for x in tr.seq_lens))
    out = torch.empty(B, Hq, D, device=dev, dtype=torch.float32)
    wsb = pa.paged_attn_decode_workspace_size(B, Hq, Hkv, D, bs, max_len, 0)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

    # a plan per decode step (the tables change every step), shared by its layers
    psize = max(pa.paged_attn_decode_plan_size(B, Hq, Hkv, D, bs, t.shape[1], max_len, 0, pa.PA_BF16)
                for t in tr.tables)
    use_plan = not args.no_plan and psize > 0
    plan = torch.empty(max(psize, 1), dtype=torch.uint8, device=dev)

    def step(s, l):
        if l == 0 and use_plan:
            pa.paged_attn_decode_plan(plan, K[0], bt[s], sl[s], Hq, max_len, 0)
        if len(tr.copies[s]):
            pa.block_copy(K[l], V[l], pairs[s])
        pa.kv_cache_write(newk, newv, K[l], V[l], slots[s])
        if use_plan:
            pa.paged_attn_decode_planned(out, q, K[l], V[l], plan, bt[s], sl[s], tr.scale, max_len, 0, ws)
        else:
            pa.paged_attn_decode(out, q, K[l], V[l], bt[s], sl[s], tr.scale, max_len, 0, ws)

    # eager pass of the whole trace; layer 0's last decode against the oracle's replay
    for s in range(S):
        for l in range(layers):
            step(s, l)
            if l == 0 and s == S - 1:
                torch.cuda.synchronize()
                gpu_last = out.double().cpu().numpy()
    hk, hv = host_copy(torch, newk), host_copy(torch, newv)
    for s in range(S):
        if len(tr.copies[s]):
            oracle.block_copy(k0, v0, tr.copies[s])
        oracle.kv_cache_write(hk, hv, k0, v0, tr.slots[s])
    sel = np.concatenate([np.arange(0, 64, 5), np.arange(64, 96, 3), np.arange(96, B, 4)])
    ref = oracle.paged_decode(host_copy(torch, q)[sel], k0, v0, tr.tables[-1][sel], tr.seq_lens[-1][sel], tr.scale)
    err = float(np.max(np.abs(gpu_last[sel] - ref)))
    if err > 2e-3:
        raise SystemExit("bench.py: mixed-mode decode differs from the oracle (%.3e)" % err)

    def trace():
        for s in range(S):
            for l in range(layers):
                step(s, l)
    trace()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        trace()
    reps = max(1, min(args.steps, 5))
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / (reps * S)
    # the copies alone, same graph treatment
    gc = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gc):
        for s in range(S):
            if len(tr.copies[s]):
                for l in range(layers):
                    pa.block_copy(K[l], V[l], pairs[s])
    gc.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        gc.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_copy = e0.elapsed_time(e1) / (reps * S)
    n_copies = sum(len(c) for c in tr.copies)
    kv_row = Hkv * D * 2 * 2                         # K + V bytes of one token, one layer
    logical = sum(int(x.astype(np.int64).sum()) for x in tr.seq_lens) / S * kv_row
    step_bytes = layers * (logical + B * Hq * D * (2 + 4) + B * kv_row * 2 + n_copies / S * 2 * 2 * Hkv * bs * D * 2)
    return {
        "metric": METRIC, "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": reps * S, "warmup": 2, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": tr.dtype, "data": "synthetic",
        "config": {"workload": tr.name, "batch": B, "beam_groups": 16, "beam_width": 4, "sample_groups": 8,
                   "samples": 4, "greedy_rows": 32, "decode_steps": S, "layers": layers, "block_size": bs,
                   "num_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "num_blocks_per_layer": tr.num_blocks},
        "cow": {"copies": n_copies, "copied_tokens": n_copies * bs,
                "whole_copy_tokens": tr.whole_copy_tokens,
                "copy_us_per_step_all_layers": round(ms_copy * 1e3, 3)},
        "query_tokens_per_s_per_layer": round(B / (ms_step * 1e-3 / layers), 1),
        "parity_max_abs_err_sampled_rows": err, "cpu_baseline": None, "timing": "hip-graph",
        "decode_plan": "one plan per step, shared by the layers" if use_plan else None,
    }


def bench_swap(args, torch, pa, W):
    """Swap one 4K-token sequence (Llama-3.1-8B shape, 32 layers) out to pinned host memory and back
    in, with kv_swap_out / kv_swap_in (one gather kernel + one DMA copy per layer), against one
    DMA copy per block (the per-copy cost model of the pages)."""
    import synth
    dev = "cuda"
    layers = args.layers or 32
    Hkv, D, bs, tokens = 8, 128, 16, 4096
    nblk = tokens // bs
    NB = 4 * nblk
    shape = (NB, Hkv, bs, D)
    K = [W.device_values(shape, 0.5, 7000 + 2 * l, "bf16") for l in range(layers)]
    V = [W.device_values(shape, 0.5, 7001 + 2 * l, "bf16") for l in range(layers)]
    perm = synth.shuffled_block_ids(NB, 77)
    ids_out = torch.from_numpy(np.asarray(perm[:nblk], np.int64)).to(dev)
    ids_in = torch.from_numpy(np.asarray(perm[nblk:2 * nblk], np.int64)).to(dev)
    blk = Hkv * bs * D * 2                       # bytes of one block of K (or V), one layer
    per_layer = nblk * 2 * blk
    host = torch.empty(layers * per_layer, dtype=torch.uint8, pin_memory=True)
    staging = torch.empty(per_layer, dtype=torch.uint8, device=dev)

    def swap(out):
        for l in range(layers):
            h = host[l * per_layer:(l + 1) * per_layer]
            if out:
                pa.kv_swap_out(K[l], V[l], ids_out, h, staging)
            else:
                pa.kv_swap_in(K[l], V[l], ids_in, h, staging)

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps, (time.perf_counter() - w0) * 1e3 / reps

    reps = max(1, min(args.steps, 10))
    ms_out, wall_out = timed(lambda: swap(True), reps)
    ms_in, wall_in = timed(lambda: swap(False), reps)
    # the blocks that went out came back, into other physical blocks, bit for bit
    ok = all(torch.equal(K[l][ids_in], K[l][ids_out]) and torch.equal(V[l][ids_in], V[l][ids_out])
             for l in range(layers))
    if not ok:
        raise SystemExit("bench.py: swapped-in blocks differ from the swapped-out ones")
    # one DMA copy per block per layer and per K / V (layers x 2 x blocks copies)
    hv = host.view(layers, nblk, 2, blk)
    ids_h = perm[:nblk]

    def per_block():
        for l in range(layers):
            kb, vb = K[l].view(torch.uint8).view(NB, blk), V[l].view(torch.uint8).view(NB, blk)
            for i, b in enumerate(ids_h):
                hv[l, i, 0].copy_(kb[b], non_blocking=True)
                hv[l, i, 1].copy_(vb[b], non_blocking=True)
    ms_pb, wall_pb = timed(per_block, 1)
    total = layers * per_layer
    copies = layers * 2 * nblk
    link = total / (ms_out * 1e-3)
    model = synth.swap_time_model(tokens, bs, layers, Hkv, D, 2, link, 0.0)
    return {
        "metric": "swap of one 4K-token sequence's KV blocks between HBM and pinned host memory, ms",
        "value": round(ms_out, 3), "unit": "ms (swap-out, 32 layers)", "n_gpus": 1, "steps": reps,
        "warmup": 2, "ms_per_step": round(ms_out, 3), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "swap_llama8b_4k", "tokens": tokens, "block_size": bs, "num_kv_heads": Hkv,
                   "head_dim": D, "layers": layers, "bytes_each_way": total, "staging_bytes": per_layer},
        "swap_out_ms": round(ms_out, 3), "swap_in_ms": round(ms_in, 3),
        "swap_out_GBs": round(total / (ms_out * 1e-3) / 1e9, 2),
        "swap_in_GBs": round(total / (ms_in * 1e-3) / 1e9, 2),
        "host_wall_ms_out_in": [round(wall_out, 3), round(wall_in, 3)],
        "per_block_copies": {"copies": copies, "ms": round(ms_pb, 3), "host_wall_ms": round(wall_pb, 3),
                             "overhead_us_per_copy": round((ms_pb - model[2] * 1e3) * 1e3 / copies, 3)},
        "pages_estimate_ms": 16.0, "round_trip_bit_exact": ok, "cpu_baseline": None,
    }


def bench_copy(args, torch):
    """A plain device copy of known size: the reference for scaling the HBM byte counters."""
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    x.fill_(1)
    y = torch.empty_like(x)
    for _ in range(args.warmup):
        y.copy_(x)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        y.copy_(x)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    return {"workload": "copy_calibration", "bytes_read_per_copy": n, "bytes_written_per_copy": n,
            "ms_per_copy": round(ms, 4), "copy_GBs_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only (no collectives or sharding are part of it); "
              "got --gpus %d, WORLD_SIZE %d" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    import torch
    import paged_kv_cache_attn_amd as pa
    from synth import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    fp8 = args.workload.endswith("_fp8")
    if args.workload in ("llama8b_decode", "llama8b_decode_fp8"):
        w = W.llama8b_decode(block_size=args.block_size)
        layers = args.layers or 32
        part = 0 if args.partition < 0 else args.partition
        res = bench_decode(args, torch, pa, W, w, layers, part, fp8=fp8)
    elif args.workload in ("tiny_decode", "llama8b_decode_f32"):
        w = W.tiny_decode() if args.workload == "tiny_decode" else W.llama8b_decode(dtype="f32")
        layers = args.layers or 32
        part = 0 if args.partition < 0 else args.partition
        res = bench_decode(args, torch, pa, W, w, layers, part)
    elif args.workload in ("llama70b_long", "llama70b_long_fp8", "llama70b_one_long"):
        w = W.llama70b_long(block_size=args.block_size) if args.workload != "llama70b_one_long" else W.llama70b_one_long()
        layers = args.layers or 4
        part = 0 if args.partition < 0 else args.partition
        res = bench_decode(args, torch, pa, W, w, layers, part, fp8=fp8)
    elif args.workload in ("chunked_prefill", "chunked_prefill_fp8"):
        w = W.chunked_prefill(block_size=args.block_size)
        res = bench_prefill(args, torch, pa, W, w, args.layers or 32, fp8=fp8)
    elif args.workload in ("shared_prefix", "shared_prefix_cow"):
        w = W.shared_prefix(prompt_len=512 if args.workload == "shared_prefix" else 500)
        res = bench_shared_prefix(args, torch, pa, W, w, args.layers or 32)
    elif args.workload == "block_size_sweep":
        res = bench_block_sizes(args, torch, pa, W)
    elif args.workload == "mixed_decode":
        res = bench_mixed_decode(args, torch, pa, W)
    elif args.workload == "swap":
        res = bench_swap(args, torch, pa, W)
    elif args.workload == "copy_calibration":
        res = bench_copy(args, torch)
    elif args.workload in ("llama8b_decode_timeline", "llama70b_long_timeline"):
        w = W.llama8b_decode() if args.workload.startswith("llama8b") else W.llama70b_long()
        res = bench_decode_timeline(args, torch, pa, W, w, args.layers or (32 if args.workload.startswith("llama8b")
                                                                            else 4))
    else:
        raise SystemExit("workload %s: not wired into the bench yet" % args.workload)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
