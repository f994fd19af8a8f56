#!/usr/bin/env python3
"""Throughput of the Flash-MoE expert layer on one MI355X.

A step is one pass of the whole layer (RMSNorm, router GEMV, softmax/top-K,
fused gate+up dequant GEMV + SwiGLU for the K selected experts and the shared
expert, down-projection with weighted combine, sigmoid-gated shared expert and
residual) over one batch of synthetic tokens, through the C ABI.

Workloads (``--workload``):
  layer4   (default) the single-token layer of hidden 4096, FFN 1024, 512 4-bit
           experts + 1 shared, top-4.  32 independent layers (32 x 3.6 GB) are
           resident and steps rotate over them and over a pool of 1024 tokens,
           so consecutive steps do not re-read the same experts from cache.
  layer2   the same layer with 2-bit experts.
  tiny     hidden 256, FFN 128, 8 experts, top-2 (latency-bound: also reports
           the median microseconds of one call).
  batch32  32 tokens with top-10, grouped by expert.
  stack60  60 chained 4-bit layers resident in HBM (218 GB); a step is one
           token through all 60 layers, one moe_stack_forward call.
  tier4    tiered expert residency (experts in pinned host memory).
  gdn      the GatedDeltaNet recurrent-state update of the linear-attention
           layers: 64 heads x 128 x 128 fp32 state, one token per step.
  stream, gap, exchange   measurement kernels of the library: HBM streaming
           read rate, dependent kernel boundaries, grid-wide exchanges.

Per-kernel durations are marginal: for each stage s, a HIP graph of M steps
that run stages 0..s is timed between two events on its stream, and stage s
is charged the difference from the graph of stages 0..s-1.  Each kernel thus
runs as in the full layer (inputs just written by the kernel before it), and
the durations add up to the time of a step.

Prints one JSON line.  `value` is tokens/s with all inputs resident in HBM.
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

HBM_PEAK_BPS = 8.0e12  # MI355X HBM3E peak
METRIC = "MoE-layer decode tokens/s (effective expert-weight HBM GB/s and % of peak alongside)"

# HBM traffic per launch of the expert kernels, keyed by (workload, kernel),
# from rocprofv3 FETCH_SIZE / WRITE_SIZE runs (summaries under profiles/); an
# entry holds only while the kernel sources hash to the prefix it was measured
# on.  FETCH_SIZE is scaled by 2.0 and WRITE_SIZE by 1.0, the ratios of bytes
# moved to counts reported for a 256 MiB copy.
KERNEL_TRAFFIC = {
    ("layer4", "k_gateup"): {"source_sha256_prefix": "02152d97d7a87fca", "fetch_kib": 11625.28125, "write_kib": 40.125,
                             "fetch_scale": 2.0, "write_scale": 1.0},
    ("layer4", "k_down"): {"source_sha256_prefix": "02152d97d7a87fca", "fetch_kib": 5907.5, "write_kib": 16.0,
                           "fetch_scale": 2.0, "write_scale": 1.0},
    ("layer2", "k_gateup"): {"source_sha256_prefix": "02152d97d7a87fca", "fetch_kib": 6514.0625, "write_kib": 20.125,
                             "fetch_scale": 2.0, "write_scale": 1.0},
    ("layer2", "k_down"): {"source_sha256_prefix": "02152d97d7a87fca", "fetch_kib": 3347.0, "write_kib": 16.0,
                           "fetch_scale": 2.0, "write_scale": 1.0},
    ("batch32", "k_grouped_gateup"): {"source_sha256_prefix": "2ab152e68fa0c42b", "fetch_kib": 569578.6875,
                                      "write_kib": 3621.21875, "fetch_scale": 2.0, "write_scale": 1.0},
    ("batch32", "k_grouped_down"): {"source_sha256_prefix": "2ab152e68fa0c42b", "fetch_kib": 287705.8125,
                                    "write_kib": 6141.5, "fetch_scale": 2.0, "write_scale": 1.0},
    ("gdn", "k_gdn"): {"source_sha256_prefix": "aadb9822606e2f30", "fetch_kib": 2350.0, "write_kib": 4128.0,
                       "fetch_scale": 2.0, "write_scale": 1.0},
}

DEFAULT_STEPS = {"layer4": 2048, "layer2": 2048, "tiny": 2048, "batch32": 256, "stack60": 64, "tier4": 512,
                 "gdn": 2048, "stream": 100, "gap": 200, "exchange": 200}
LAYER_WORKLOADS = ("layer4", "layer2", "tiny", "batch32")
MICRO_WORKLOADS = ("stream", "gap", "exchange")


def source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_dequant_expert_router_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_source_hash(grouped):
    """sha256 of the sources the expert kernels are built from."""
    return source_hash(["moe_device.h", "moe_internal.h", "moe_layout.h",
                        "moe_grouped.hip" if grouped else "moe_forward.hip"])


def gdn_source_hash():
    """sha256 of the sources the GatedDeltaNet kernel is built from."""
    return source_hash(["moe_device.h", "moe_gdn.hip"])


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None, help="timed steps (default: per workload)")
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--workload", default="layer4",
                   choices=list(LAYER_WORKLOADS) + ["stack60", "tier4", "gdn"] + list(MICRO_WORKLOADS))
    p.add_argument("--tier-cache", type=float, default=0.71,
                   help="tier4: device slots as a fraction of the layers' experts")
    p.add_argument("--layers", type=int, default=32, help="resident layers the steps rotate over")
    p.add_argument("--pool", type=int, default=1024, help="distinct tokens the steps rotate over")
    p.add_argument("--tokens", type=int, default=0,
                   help="tokens per step (0: the workload's own; other values are for batch-size sweeps)")
    p.add_argument("--mode", default="graph", choices=["graph", "api"],
                   help="graph: the timed steps are one captured HIP graph; api: one ABI call per step")
    p.add_argument("--cpu-sample", type=int, default=24, help="tokens for the oracle CPU baseline (0: skip)")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="before timing, copy a buffer of this many MiB 8 times (a kernel of known traffic "
                        "for scaling profiler byte counters)")
    p.add_argument("--no-stages", action="store_true",
                   help="skip the per-kernel timing graphs and the roofline (for profiler runs)")
    p.add_argument("--quiet", action="store_true")
    a = p.parse_args(argv)
    if a.steps is None:
        a.steps = DEFAULT_STEPS[a.workload]
    return a


def log(args, msg):
    if not args.quiet:
        print(msg, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------- #
# algorithmic bytes (host only; tested on the CPU)
# --------------------------------------------------------------------------- #
def matrix_bytes(dims) -> int:
    """Codes and scale/bias of one expert matrix (gate, up or down)."""
    return dims.ffn * dims.hidden * dims.bits // 8 + (dims.ffn * dims.hidden // 64) * 4


def distinct_experts(idx) -> int:
    """Experts one step reads: the distinct selected ones plus the shared one.
    idx: the step's route indices [tokens][K]; every entry must be routed."""
    import numpy as np
    a = np.asarray(idx).ravel()
    if a.size == 0 or int(a.min()) < 0:
        raise ValueError("route indices of an unrouted step")
    return len(np.unique(a)) + 1


def stage_bytes(dims, names, n_distinct: float, n_tokens: int):
    """Algorithmic HBM bytes of each stage of one step: weights (router, or the
    gate/up or down matrices of the n_distinct experts read) plus the
    activations a stage must read.  Stages that read no weights get None."""
    H, E = dims.hidden, dims.n_experts
    router = (E + 1) * H * 2 + H * 2 + n_tokens * H * 4  # router rows, shared gate, gamma, x
    out = []
    for n in names:
        if n in ("k_router", "k_router_mfma"):
            out.append(router)
        elif n in ("k_gateup", "k_grouped_gateup"):
            out.append(n_distinct * 2 * matrix_bytes(dims))
        elif n in ("k_down", "k_grouped_down"):
            out.append(n_distinct * matrix_bytes(dims))
        else:
            out.append(None)
    return out


def roofline_entry(name, nbytes, seconds):
    if nbytes is None or seconds <= 0:
        return None
    ach = nbytes / seconds
    return {"kernel": name, "bound": "hbm", "achieved": round(ach / 1e9, 1), "peak": HBM_PEAK_BPS / 1e9,
            "unit": "GB/s", "frac": round(ach / HBM_PEAK_BPS, 4), "bytes_per_launch": round(nbytes),
            "launch_us": round(seconds * 1e6, 3)}


def stage_names(n_stages):
    if n_stages == 7:
        return ["k_norm_batch", "k_router_mfma", "k_route_tokens", "k_grouped_gateup", "k_encode_act",
                "k_grouped_down", "k_combine"]
    return ["k_router", "k_gateup", "k_down"]


def traffic_of(wl_name, kernel, sha):
    """Measured HBM bytes per launch, or None when the sources (hash `sha`)
    have changed since the counters were taken."""
    tr = KERNEL_TRAFFIC.get((wl_name, kernel))
    if tr is not None and tr["source_sha256_prefix"] == sha[:16]:
        return round((tr["fetch_kib"] * tr["fetch_scale"] + tr["write_kib"] * tr["write_scale"]) * 1024)
    return None


def refuse_multi_gpu(args):
    if args.gpus != 1:
        msg = (f"bench.py: --gpus {args.gpus} is not supported: the library runs the expert layer on one GPU "
               "(every expert resident in that GPU's HBM); run with --gpus 1")
        print(msg, flush=True)
        print(msg, file=sys.stderr, flush=True)
        sys.exit(2)


def main(argv=None):
    args = parse_args(argv)
    refuse_multi_gpu(args)
    if args.workload in MICRO_WORKLOADS:
        return bench_micro(args)
    if args.workload == "gdn":
        return bench_gdn(args)
    import synthetic as syn
    wl = syn.WORKLOADS[args.workload]
    if wl.name == "tier4":
        return bench_tier(args, wl)
    if wl.name == "stack60":
        return bench_stack(args, wl)
    return bench_layer(args, wl)


def graph_of(fn):
    """A HIP graph capturing fn() on a side stream."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    return g


def time_replay(g, reps=2):
    """Best elapsed seconds of `reps` replays of graph g, between events on the
    stream the replay runs on."""
    import torch
    g.replay()
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        # replay() launches the graph on the current stream: the events bracket it there
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        el = e0.elapsed_time(e1) * 1e-3
        best = el if best is None else min(best, el)
    return best


def marginal_stages(n_stages, M, launch_stage):
    """Per-stage seconds: graph(stages 0..s) minus graph(stages 0..s-1), per step.
    launch_stage(i, st) enqueues stage st of step i."""
    import numpy as np
    prefix = []
    for last in range(n_stages):
        g = graph_of(lambda: [launch_stage(i, st) for i in range(M) for st in range(last + 1)])
        prefix.append(time_replay(g) / M)
        del g
    return np.diff(np.array([0.0] + prefix))


# --------------------------------------------------------------------------- #
# single layers and batches
# --------------------------------------------------------------------------- #
def bench_layer(args, wl):
    import numpy as np
    import torch

    import bit_dequant_expert_router_amd as moe
    import synthetic as syn
    from bit_dequant_expert_router_amd.weights import layer_generated

    dims = wl.dims
    T = args.tokens if args.tokens > 0 else wl.n_tokens
    K = dims.top_k
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    R = max(1, args.layers)
    log(args, f"[bench] {wl.name}: {wl.description}; generating {R} layers on the device")
    layers = [layer_generated(dims, syn.layer_dense(wl.seed, l, dims), wl.seed, l, device=dev) for l in range(R)]
    descs = [lw.descriptor() for lw in layers]
    P = max(1, args.pool)
    pool = torch.from_numpy(syn.tokens(wl.seed, P * T, dims.hidden).reshape(P, T, dims.hidden)).to(dev)
    out = torch.empty_like(pool)
    ridx = torch.full((P, T, K), -1, dtype=torch.int32, device=dev)
    rw = torch.empty((P, T, K), dtype=torch.float32, device=dev)
    wsb = moe.moe_workspace_bytes(dims, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    moe.moe_workspace_init(ws)
    torch.cuda.synchronize()

    def step(i):
        j = i % P
        moe.moe_layer_forward(dims, descs[i % R], pool[j], out[j], T, ridx[j], rw[j], ws, wsb)

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region
    nsteps = args.steps
    graph = None
    if args.mode == "graph":
        graph = graph_of(lambda: [step(i) for i in range(nsteps)])
        graph.replay()  # warm replay
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for i in range(nsteps):
            step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    del graph
    ms_per_step = elapsed * 1e3 / nsteps
    tokens_per_s = nsteps * T / elapsed

    if args.no_stages:
        print(json.dumps({"metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
                          "steps": nsteps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
                          "note": "profiler run: no per-kernel timing, no roofline"}), flush=True)
        return

    # per-kernel durations, marginal: NW steps (token j, layer j mod R) get a
    # workspace each, filled by one full forward
    NW = min(P, 64)
    wss = [torch.empty(wsb, dtype=torch.uint8, device=dev) for _ in range(NW)]
    for w in wss:
        moe.moe_workspace_init(w)
    for j in range(NW):
        moe.moe_layer_forward(dims, descs[j % R], pool[j], out[j], T, ridx[j], rw[j], wss[j], wsb)
    torch.cuda.synchronize()

    # algorithmic expert-weight bytes from the routes the timed steps (rows
    # i mod P) and the stage steps (rows 0..NW-1) wrote: every row read here
    # has been written by then
    idx_all = ridx.cpu().numpy()
    eb = moe.moe_expert_bytes(dims)
    steps_rows = sorted({i % P for i in range(nsteps)})
    distinct = {j: distinct_experts(idx_all[j]) for j in set(steps_rows) | set(range(NW))}
    bytes_total = float(sum(distinct[i % P] for i in range(nsteps))) * eb
    bytes_per_step = bytes_total / nsteps
    router_bytes = dims.n_experts * dims.hidden * 2

    n_stages = moe.moe_forward_stage_count(dims, T)
    grouped = n_stages == 7
    names = stage_names(n_stages)
    M = 64 if grouped else 512

    def launch_stage(i, st):
        j = i % NW
        moe.moe_layer_forward_stage(dims, descs[j % R], pool[j], out[j], T, ridx[j], rw[j], wss[j], wsb, st)

    stage_s = marginal_stages(n_stages, M, launch_stage)
    n_distinct = float(np.mean([distinct[j] for j in range(NW)]))
    sbytes = stage_bytes(dims, names, n_distinct, T)
    stages = [roofline_entry(n, b, s) for n, b, s in zip(names, sbytes, stage_s)]
    # the dominant expert kernel: the longest of gate/up and down
    expert_stages = [k for k, n in enumerate(names) if "gateup" in n or "down" in n]
    dom = max(expert_stages, key=lambda k: stage_s[k])
    roof = dict(stages[dom])
    roof["traffic"] = (traffic_of(wl.name, names[dom], kernel_source_hash(grouped))
                       if T == wl.n_tokens else None)

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": nsteps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: {wl.description}" if T == wl.n_tokens else
                        f"{wl.name} shape at {T} tokens per step: {wl.description}",
            "hidden": dims.hidden, "ffn": dims.ffn, "n_experts": dims.n_experts, "top_k": K,
            "bits": dims.bits, "group_size": dims.group_size, "tokens_per_step": T,
            "resident_layers": R, "token_pool": P, "mode": args.mode,
        },
        "expert_bytes_per_step": round(bytes_per_step),
        "router_bytes_per_step": router_bytes,
        "effective_expert_GBps": round(bytes_per_step * nsteps / elapsed / 1e9, 1),
        "pct_of_hbm_peak": round(100.0 * bytes_per_step * nsteps / elapsed / HBM_PEAK_BPS, 2),
        "roofline": roof,
        "stage_us": {n: round(float(v) * 1e6, 3) for n, v in zip(names, stage_s)},
        "stage_roofline": [s for s in stages if s is not None],
    }
    if wl.name == "tiny":
        result["us_per_call_p50"] = call_latency_p50(moe, dims, descs, pool, out, ridx, rw, ws, wsb, T, R, P)

    if args.cpu_sample > 0:
        result["cpu_baseline"] = cpu_baseline(args, wl, dims)

    print(json.dumps(result), flush=True)


def call_latency_p50(moe, dims, descs, pool, out, ridx, rw, ws, wsb, T, R, P, n=1000, warm=50):
    """Median microseconds of one moe_layer_forward call: an event pair around
    each of n calls (after warm calls), issued one at a time.  The calls' arguments
    are marshalled before the loop (layer_forward_call), so that the figure is the
    C ABI call's, as a C caller sees it, and not Python's tensor indexing."""
    import numpy as np
    import torch
    calls = [moe.layer_forward_call(dims, descs[i % R], pool[i % P], out[i % P], T, ridx[i % P], rw[i % P], ws, wsb)
             for i in range(warm + n)]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(warm + n):
        if i >= warm:
            ev[i - warm][0].record()
        calls[i]()
        if i >= warm:
            ev[i - warm][1].record()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return round(float(np.median(us)), 3)


# --------------------------------------------------------------------------- #
# the 60-layer stack
# --------------------------------------------------------------------------- #
def bench_stack(args, wl):
    import numpy as np
    import torch

    import bit_dequant_expert_router_amd as moe
    import synthetic as syn
    from bit_dequant_expert_router_amd.weights import layer_generated

    dims = wl.dims
    L, K = wl.n_layers, dims.top_k
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    log(args, f"[bench] {wl.name}: {wl.description}; generating {L} layers on the device")
    dense = [syn.layer_dense(wl.seed, l, dims) for l in range(L)]
    layers = [layer_generated(dims, dense[l], wl.seed, l, device=dev) for l in range(L)]
    descs = [lw.descriptor() for lw in layers]
    eb = moe.moe_expert_bytes(dims)
    resident = L * (dims.n_experts + 1) * eb + L * dims.n_experts * dims.hidden * 2
    P = min(max(1, args.pool), 64)
    pool = torch.from_numpy(syn.tokens(wl.seed, P, dims.hidden).reshape(P, 1, dims.hidden)).to(dev)
    out = torch.empty_like(pool)
    ridx = torch.full((P, L, 1, K), -1, dtype=torch.int32, device=dev)
    rw = torch.empty((P, L, 1, K), dtype=torch.float32, device=dev)
    wsb = moe.moe_workspace_bytes(dims, 1)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    moe.moe_workspace_init(ws)
    torch.cuda.synchronize()

    def step(i):
        j = i % P
        moe.moe_stack_forward(dims, descs, pool[j], out[j], 1, ridx[j], rw[j], ws, wsb)

    for i in range(min(args.warmup, 8)):
        step(i)
    torch.cuda.synchronize()
    nsteps = args.steps
    graph = None
    if args.mode == "graph":
        graph = graph_of(lambda: [step(i) for i in range(nsteps)])
        graph.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for i in range(nsteps):
            step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    del graph
    if args.no_stages:
        print(json.dumps({"metric": METRIC, "value": round(nsteps / elapsed, 2), "unit": "tokens/s",
                          "n_gpus": 1, "steps": nsteps, "ms_per_step": round(elapsed * 1e3 / nsteps, 6),
                          "note": "profiler run: no per-kernel timing, no roofline"}), flush=True)
        return
    idx_all = ridx.cpu().numpy()
    rows = sorted({i % P for i in range(nsteps)})
    per_token = {j: sum(distinct_experts(idx_all[j, l]) for l in range(L)) * eb for j in rows}
    bytes_total = float(sum(per_token[i % P] for i in range(nsteps)))

    # per-stage durations over chained layers: M tokens x L layers, each layer
    # reading the stack's running state (y) as moe_stack_forward does
    M = 4
    n_stages = moe.moe_forward_stage_count(dims, 1)
    names = stage_names(n_stages)

    def launch_stage(i, st):
        j = i // L % P
        l = i % L
        moe.moe_layer_forward_stage(dims, descs[l], pool[j] if l == 0 else out[j], out[j], 1, ridx[j, l],
                                    rw[j, l], ws, wsb, st)

    stage_s = marginal_stages(n_stages, M * L, launch_stage)
    n_distinct = float(np.mean([distinct_experts(idx_all[j, l]) for j in range(min(P, M)) for l in range(L)]))
    sbytes = stage_bytes(dims, names, n_distinct, 1)
    stages = [roofline_entry(n, b, s) for n, b, s in zip(names, sbytes, stage_s)]
    dom = 1 if stage_s[1] >= stage_s[2] else 2
    roof = dict(stages[dom])
    # the stack runs the single layer's kernels on the same shape, one token
    # per launch: their measured traffic per launch is the single layer's
    single = {(4, 4096, 1024, 512, 4): "layer4", (2, 4096, 1024, 512, 4): "layer2"}.get(
        (dims.bits, dims.hidden, dims.ffn, dims.n_experts, dims.top_k))
    roof["traffic"] = traffic_of(single, names[dom], kernel_source_hash(False)) if single else None

    result = {
        "metric": METRIC,
        "value": round(nsteps / elapsed, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": nsteps,
        "warmup": min(args.warmup, 8),
        "ms_per_step": round(elapsed * 1e3 / nsteps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: {wl.description}",
            "hidden": dims.hidden, "ffn": dims.ffn, "n_experts": dims.n_experts, "top_k": K,
            "bits": dims.bits, "group_size": dims.group_size, "tokens_per_step": 1, "layers": L,
            "resident_bytes": resident, "token_pool": P, "mode": args.mode,
        },
        "note": "value counts tokens through all 60 layers per second (one moe_stack_forward call each)",
        "us_per_layer": round(elapsed * 1e6 / (nsteps * L), 3),
        "expert_bytes_per_step": round(bytes_total / nsteps),
        "router_bytes_per_step": L * dims.n_experts * dims.hidden * 2,
        "effective_expert_GBps": round(bytes_total / elapsed / 1e9, 1),
        "pct_of_hbm_peak": round(100.0 * bytes_total / elapsed / HBM_PEAK_BPS, 2),
        "roofline": roof,
        "stage_us": {n: round(float(v) * 1e6, 3) for n, v in zip(names, stage_s)},
        "stage_roofline": [s for s in stages if s is not None],
    }
    if args.cpu_sample > 0:
        result["cpu_baseline"] = cpu_baseline_stack(args, wl, dims, dense)
    print(json.dumps(result), flush=True)


# --------------------------------------------------------------------------- #
# measurement kernels of the library
# --------------------------------------------------------------------------- #
def bench_micro(args):
    import numpy as np
    import torch

    import bit_dequant_expert_router_amd as moe
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    R = args.steps
    base = {"n_gpus": 1, "steps": R, "warmup": 1, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "data": "synthetic"}
    if args.workload == "stream":
        # reads of contiguous buffers at rotating offsets inside 2 GiB, so that
        # consecutive reads do not hit the 256 MB memory-side cache
        big = 2 << 30
        buf = torch.empty(big, dtype=torch.uint8, device=dev).fill_(1)
        sink = torch.zeros(16, dtype=torch.uint8, device=dev)
        rows = []
        for mib in (4, 12, 35, 64, 256, 1024):
            nbytes = mib << 20
            nslot = big // nbytes
            reps = R if mib < 256 else max(4, R // 10)
            for blocks in (512, 1024, 2048):
                for fl in (1, 2, 4):
                    g = graph_of(lambda: [moe.moe_mb_stream_read(buf[(i % nslot) * nbytes:], nbytes, blocks, fl, sink)
                                          for i in range(reps)])
                    s = time_replay(g) / reps
                    rows.append({"MiB": mib, "blocks": blocks, "loads_in_flight": fl, "us": round(s * 1e6, 3),
                                 "TBps": round(nbytes / s / 1e12, 3)})
                    del g
        best = {}
        for r in rows:
            if r["MiB"] not in best or r["TBps"] > best[r["MiB"]]["TBps"]:
                best[r["MiB"]] = r
        result = dict(base, metric="HBM streaming read rate (16-byte nontemporal loads, contiguous block ranges)",
                      value=round(best[1024]["TBps"] * 1e3, 1), unit="GB/s", ms_per_step=None, dtype="u32",
                      config={"workload": "stream: reads of 4 MiB to 1 GiB at rotating offsets in 2 GiB, "
                                          "512-2048 blocks of 256 threads, 1-4 loads in flight per lane"},
                      best_per_size={str(k): v for k, v in sorted(best.items())}, table=rows)
    elif args.workload == "gap":
        rows = {}
        for blocks in (1, 256, 1024):
            g = graph_of(lambda: [moe.moe_mb_empty(blocks) for _ in range(R)])
            rows[f"empty_{blocks}_blocks_us"] = round(time_replay(g) / R * 1e6, 3)
            del g
        # three dependent streaming kernels of the layer's sizes (4, 24, 12 MiB)
        # against one stream of their sum
        big = 2 << 30
        buf = torch.empty(big, dtype=torch.uint8, device=dev).fill_(1)
        sink = torch.zeros(16, dtype=torch.uint8, device=dev)
        sizes = [4 << 20, 24 << 20, 12 << 20]
        tot = sum(sizes)
        nslot = big // tot

        def three(i):
            off = (i % nslot) * tot
            for sz in sizes:
                moe.moe_mb_stream_read(buf[off:], sz, 1024, 2, sink)
                off += sz

        g = graph_of(lambda: [three(i) for i in range(R)])
        rows["three_dependent_reads_4_24_12_MiB_us"] = round(time_replay(g) / R * 1e6, 3)
        del g
        # the same with the layer's in-kernel dependencies: the second and
        # third kernels first read a 2 KiB vector that the kernel before wrote
        # (as the logits and the selection are), and only then their bytes
        vec = torch.zeros(3, 2048, dtype=torch.uint8, device=dev)
        nslot_d = (big - (64 << 10)) // tot

        def three_dep(i):
            off = (i % nslot_d) * tot
            moe.moe_mb_dependent_read(buf[off:], sizes[0], 1024, 2, None, vec[0], sink)
            off += sizes[0]
            moe.moe_mb_dependent_read(buf[off:], sizes[1], 1024, 2, vec[0], vec[1], sink)
            off += sizes[1]
            moe.moe_mb_dependent_read(buf[off:], sizes[2], 1024, 2, vec[1], vec[2], sink)

        g = graph_of(lambda: [three_dep(i) for i in range(R)])
        rows["three_dependent_reads_with_vector_reads_us"] = round(time_replay(g) / R * 1e6, 3)
        del g
        g = graph_of(lambda: [moe.moe_mb_stream_read(buf[(i % nslot) * tot:], tot, 1024, 2, sink) for i in range(R)])
        rows["one_read_40_MiB_us"] = round(time_replay(g) / R * 1e6, 3)
        del g
        result = dict(base, metric="dependent kernel boundary inside a HIP graph",
                      value=rows["empty_256_blocks_us"], unit="us per empty kernel", higher_is_better=False,
                      ms_per_step=None, dtype="none",
                      config={"workload": "gap: chains of empty kernels (1, 256, 1024 blocks) in one graph; "
                                          "three dependent reads of 4 + 24 + 12 MiB, also with each read behind a "
                                          "2 KiB vector the previous kernel wrote, against one 40 MiB read"},
                      **rows)
    else:  # exchange
        rows = []
        g = graph_of(lambda: [moe.moe_mb_empty(256) for _ in range(R)])
        empty_us = time_replay(g) / R * 1e6
        del g
        fails = 0
        cases = [(kind, blocks, groups) for kind in (0, 1, 2, 3) for blocks in (256, 512) for groups in (1, 8, 32)]
        cases += [(4, blocks, groups) for blocks in (512, 1024, 1152) for groups in (8, 32)]
        names = {0: "arrivals", 1: "barrier", 2: "barrier, replicated release", 3: "all-to-all tagged words",
                 4: "producers then consumers"}
        for kind, blocks, groups in cases:
            nb = moe.moe_mb_exchange_bytes(blocks, groups)
            buf = torch.zeros(nb, dtype=torch.uint8, device=dev)
            g = graph_of(lambda: [moe.moe_mb_exchange(kind, blocks, groups, buf) for _ in range(R)])
            us = time_replay(g) / R * 1e6
            f = moe.moe_mb_exchange_failures(buf)
            fails += f
            rows.append({"kind": kind, "pattern": names[kind], "blocks": blocks, "groups": groups,
                         "us": round(us, 3), "over_empty_kernel_us": round(us - empty_us, 3), "gave_up": f})
            del g, buf
        result = dict(base, metric="grid-wide exchange inside one kernel",
                      value=round(min(r["over_empty_kernel_us"] for r in rows if r["kind"] == 1), 3),
                      unit="us over an empty kernel (best grid barrier)", higher_is_better=False,
                      ms_per_step=None, dtype="none",
                      config={"workload": "exchange: arrivals, two-level grid barriers and an all-to-all of "
                                          "tagged words over 256 and 512 blocks, 1-32 first-level counters; "
                                          "producer/consumer halves of 512-1152 blocks"},
                      empty_kernel_us=round(empty_us, 3), waits_given_up=fails, table=rows)
    print(json.dumps(result), flush=True)


# --------------------------------------------------------------------------- #
# GatedDeltaNet state update
# --------------------------------------------------------------------------- #
def gdn_step_bytes(n_heads, d, T=1):
    """Algorithmic HBM bytes of one call: the fp32 state read and written once,
    q, k, v, the output and the two gates per token."""
    return 2 * n_heads * d * d * 4 + T * n_heads * (4 * d * 4 + 2 * 4)


def bench_gdn(args):
    """One token per step through one layer's 64 x 128 x 128 state; the steps
    rotate over --layers states (default 128: 512 MiB, more than the 256 MB
    memory-side cache) and a pool of tokens."""
    import numpy as np
    import torch

    import bit_dequant_expert_router_amd as moe
    import synthetic as syn
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    Hh, D = 64, 128
    L = args.layers if args.layers != 32 else 128
    P = min(max(1, args.pool), 256)
    log(args, f"[bench] gdn: {Hh} heads x {D} x {D} fp32 state, {L} layer states, {P} tokens")
    x = syn.gdn_inputs(0, Hh, D, P)
    states = torch.from_numpy(np.tile(x["state"], (L, 1, 1, 1))).to(dev)
    for l in range(L):  # distinct states per layer (scaled copies)
        states[l].mul_(1.0 + 0.001 * l)
    q, k, v, alpha, beta = (torch.from_numpy(x[n]).to(dev) for n in ("q", "k", "v", "alpha", "beta"))
    out = torch.empty((P, Hh, D), dtype=torch.float32, device=dev)

    def step(i):
        j = i % P
        moe.moe_gdn_update(Hh, D, D, 1, states[i % L], q[j], k[j], v[j], alpha[j], beta[j], out[j])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    nsteps = args.steps
    g = graph_of(lambda: [step(i) for i in range(nsteps)])
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # the kernel's own time, between events around a graph of the same launches
    launch_s = time_replay(g) / nsteps
    nb = gdn_step_bytes(Hh, D)
    roof = roofline_entry("k_gdn", nb, launch_s)
    roof["traffic"] = traffic_of("gdn", "k_gdn", gdn_source_hash())
    result = {
        "metric": "GatedDeltaNet state updates per second (one token through one layer) and state GB/s",
        "value": round(nsteps / elapsed, 1),
        "unit": "layer-tokens/s",
        "n_gpus": 1,
        "steps": nsteps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / nsteps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"gdn: {Hh} heads x {D} x {D} fp32 state, one token per step, {L} layer states",
                   "n_heads": Hh, "d_k": D, "d_v": D, "layer_states": L, "token_pool": P, "mode": "graph"},
        "bytes_per_step": nb,
        "effective_GBps": round(nb * nsteps / elapsed / 1e9, 1),
        "pct_of_hbm_peak": round(100.0 * nb * nsteps / elapsed / HBM_PEAK_BPS, 2),
        "roofline": roof,
    }
    if args.cpu_sample > 0:
        import oracle.gdn as og
        xs = [{n: x[n][j:j + 1] for n in ("q", "k", "v", "alpha", "beta")} for j in range(min(P, 8))]
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 1.5:
            j = done % len(xs)
            og.gdn_layer(x["state"], xs[j]["q"], xs[j]["k"], xs[j]["v"], xs[j]["alpha"], xs[j]["beta"])
            done += 1
        el = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(done / el, 3), "unit": "layer-tokens/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": f"{done} single-token updates of the {Hh}-head state, fp64 numpy "
                                            f"oracle (one head at a time), {el:.1f} s wall"}
    print(json.dumps(result), flush=True)


PCIE5_X16_BPS = 64.0e9  # MI355X host link, PCIe 5.0 x16, per direction


def bench_tier(args, wl):
    """Tiered residency: wl.n_layers chained layers whose experts live in pinned
    host memory, a device cache of --tier-cache of them.  A step is one token
    through every layer; `value` counts layer passes per second, like the
    resident workloads."""
    import numpy as np
    import torch

    import bit_dequant_expert_router_amd as moe
    import synthetic as syn
    from bit_dequant_expert_router_amd.weights import layer_generated

    dims = wl.dims
    K, E, L = dims.top_k, dims.n_experts, wl.n_layers
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    eb = moe.moe_expert_bytes(dims)
    n_slots = max(K, int(round(args.tier_cache * L * E)))
    log(args, f"[bench] {wl.name}: {wl.description}; {n_slots} slots ({n_slots * eb / 1e9:.1f} GB) for "
              f"{L * E} experts; generating {L} layers")
    layers, hosts, keep = [], [], []
    for l in range(L):
        lw = layer_generated(dims, syn.layer_dense(wl.seed, l, dims), wl.seed, l, device=dev)
        h = torch.empty(lw.experts.numel(), dtype=torch.uint8, pin_memory=True)
        h.copy_(lw.experts)
        torch.cuda.synchronize()
        lw.experts = None  # the routed experts now live in host memory only
        hosts.append(h)
        layers.append(moe.make_layer(lw.norm_weight, lw.router_weight, lw.shared_gate, h, lw.shared))
        keep.append(lw)
    state = torch.zeros(moe.moe_tier_state_bytes(dims, L, n_slots, 1), dtype=torch.uint8, pin_memory=True)
    slots = torch.empty(moe.moe_tier_device_bytes(dims, n_slots, 1), dtype=torch.uint8, device=dev)
    moe.moe_tier_init(dims, L, n_slots, 1, state, slots)
    wsb = moe.moe_workspace_bytes(dims, 1)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    moe.moe_workspace_init(ws)
    P = max(1, args.pool) * L + 1  # coprime with L: every layer meets every token of the pool
    pool = torch.from_numpy(syn.tokens(wl.seed, P, dims.hidden).reshape(P, 1, dims.hidden)).to(dev)
    out = torch.empty_like(pool)

    # for reference, the rate of plain DMA copies of one expert each (the
    # library's copy kernel, which a miss uses, reads the host memory itself)
    dst = slots[:eb]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(64):
        dst.copy_(hosts[i % L][(i * 7 % E) * eb:(i * 7 % E + 1) * eb], non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    copy_bps = 64 * eb / (e0.elapsed_time(e1) * 1e-3)

    # every layer pass takes a fresh token from the pool (as the resident
    # workloads do): chained synthetic layers would route every token alike
    # after the first layer (their random experts add a large common component
    # to the residual stream), which would flatter the cache
    def step(i):
        for l in range(L):
            j = (i * L + l) % P
            moe.moe_tier_layer_forward(state, l, layers[l], pool[j], out[j], 1, None, None, ws, wsb)

    # warm-up until every slot has been filled once (the steady state), then a
    # further --warmup steps
    nwarm = 0
    while moe.moe_tier_get_stats(state).misses < n_slots and nwarm < 100000:
        step(nwarm)
        nwarm += 1
    for _ in range(args.warmup):
        step(nwarm)
        nwarm += 1
    torch.cuda.synchronize()
    s0 = moe.moe_tier_get_stats(state)
    nsteps = args.steps
    t0 = time.perf_counter()
    for i in range(nsteps):
        step(nwarm + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    s1 = moe.moe_tier_get_stats(state)
    lookups, misses = s1.lookups - s0.lookups, s1.misses - s0.misses
    copied = s1.bytes_copied - s0.bytes_copied
    passes = nsteps * L
    link_bps = copied / elapsed
    result = {
        "metric": METRIC,
        "value": round(passes / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": nsteps,
        "warmup": nwarm,
        "ms_per_step": round(elapsed * 1e3 / nsteps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: {wl.description}",
            "hidden": dims.hidden, "ffn": dims.ffn, "n_experts": E, "top_k": K, "bits": dims.bits,
            "group_size": dims.group_size, "tokens_per_step": 1, "layers": L, "cache_slots": n_slots,
            "cache_fraction": round(n_slots / (L * E), 4), "token_pool": P, "mode": "api",
        },
        "note": "value counts layer passes (one token through one layer) per second; each pass takes a "
                "fresh token, waits for its routing on the host, then copies its missing experts and runs "
                "the expert kernels",
        "us_per_layer": round(elapsed * 1e6 / passes, 2),
        "hit_rate": round(1.0 - misses / max(lookups, 1), 4),
        "misses_per_layer": round(misses / passes, 3),
        "roofline": {
            "kernel": "k_fetch (missing experts, host memory to their slots over the host link)",
            "bound": "pcie",
            "achieved": round(link_bps / 1e9, 2),
            "peak": PCIE5_X16_BPS / 1e9,
            "unit": "GB/s",
            "frac": round(link_bps / PCIE5_X16_BPS, 4),
            "traffic": None,
            "dma_copy_GBps": round(copy_bps / 1e9, 2),
        },
    }
    print(json.dumps(result), flush=True)


# --------------------------------------------------------------------------- #
# CPU baselines: the fp64 oracle as it stands, on a bounded sample
# --------------------------------------------------------------------------- #
def cpu_baseline(args, wl, dims):
    """The fp64 oracle on a bounded sample of the same workload."""
    import oracle
    import synthetic as syn
    n = max(1, args.cpu_sample // wl.n_tokens)  # steps holding about cpu_sample tokens
    R = max(1, args.layers)
    xs = syn.tokens(wl.seed, n * wl.n_tokens, dims.hidden).reshape(n, wl.n_tokens, dims.hidden)
    cache = {}

    def fetch(layer):
        def f(e):
            key = (layer, e)
            if key not in cache:
                cache[key] = syn.expert_canonical(wl.seed, layer, e, dims)
            return cache[key]
        return f

    dense = {l: syn.layer_dense(wl.seed, l, dims) for l in range(min(R, n))}
    # routing first (untimed) so that input generation is outside the timed region
    for i in range(n):
        l = i % R % len(dense)
        for t in range(wl.n_tokens):
            h = oracle.rmsnorm(xs[i, t], dense[l]["norm_weight"], dims.rms_eps)
            idx, _ = oracle.route(oracle.gemv_bf16(dense[l]["router_weight"], h), dims.top_k)
            for e in list(idx) + [dims.n_experts]:
                fetch(l)(int(e))
    log(args, f"[bench] cpu baseline: oracle on {n} steps x {wl.n_tokens} tokens, {oracle.threads()} threads")
    # passes over the sample until about 1.5 s of wall time (x the oracle's threads of CPU work)
    done = 0
    t0 = time.perf_counter()
    while True:
        for i in range(n):
            l = i % R % len(dense)
            for t in range(wl.n_tokens):
                oracle.layer(dims, xs[i, t], dense[l], fetch(l))
        done += 1
        el = time.perf_counter() - t0
        if el >= 1.5:
            break
    return {
        "value": round(done * n * wl.n_tokens / el, 3),
        "unit": "tokens/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": f"{done} passes over {n} steps of the {wl.name} workload ({n * wl.n_tokens} tokens, "
                  f"layers rotating), fp64 C oracle, {el:.1f} s wall on {oracle.threads()} threads",
    }


def cpu_baseline_stack(args, wl, dims, dense):
    """The fp64 oracle chaining one token through the stack: a first pass
    generates the canonical experts it routes to (untimed), the second is timed."""
    import oracle
    import synthetic as syn
    L = wl.n_layers
    x0 = syn.tokens(wl.seed, 1, dims.hidden)[0]
    cache = {}

    def fetch(layer):
        def f(e):
            key = (layer, e)
            if key not in cache:
                cache[key] = syn.expert_canonical(wl.seed, layer, e, dims)
            return cache[key]
        return f

    def run():
        x = x0
        for l in range(L):
            x = oracle.layer(dims, x, dense[l], fetch(l))["out"].astype("float32")
        return x

    log(args, f"[bench] cpu baseline: oracle, one token through {L} layers, {oracle.threads()} threads")
    run()
    t0 = time.perf_counter()
    run()
    el = time.perf_counter() - t0
    return {
        "value": round(1.0 / el, 4),
        "unit": "tokens/s",
        "seconds_per_token": round(el, 3),
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": f"one token through the {L} layers (the first of the pool), fp64 C oracle, canonical "
                  f"experts generated in an untimed first pass, {el:.1f} s wall on {oracle.threads()} threads",
    }


if __name__ == "__main__":
    main()
