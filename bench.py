#!/usr/bin/env python3
"""Throughput of the Flash-MoE expert layer on one MI355X.

A step is one pass of the whole layer (RMSNorm, router GEMV, softmax/top-K,
fused gate+up dequant GEMV + SwiGLU for the K selected experts and the shared
expert, down-projection with weighted combine, sigmoid-gated shared expert and
residual) over one batch of synthetic tokens, through the C ABI.

Default workload: the single-token layer of hidden 4096, FFN 1024, 512 4-bit
experts + 1 shared, top-4.  32 independent layers (32 x 3.6 GB) are resident
and steps rotate over them and over a pool of 1024 tokens, so consecutive
steps do not re-read the same experts from cache.

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

# HBM traffic per launch of the dominant expert kernel, keyed by (workload,
# kernel), from rocprofv3 FETCH_SIZE / WRITE_SIZE runs (summaries under
# profiles/); an entry holds only while the kernel sources hash to the prefix it
# was measured on.  FETCH_SIZE is scaled by 2.0 and WRITE_SIZE by 1.0, the ratios
# of bytes moved to counts reported for a 256 MiB copy.
KERNEL_TRAFFIC = {
    ("layer4", "k_gateup"): {"source_sha256_prefix": "5271af809b8e5ad3", "fetch_kib": 11640.0, "write_kib": 20.1,
                             "fetch_scale": 2.0, "write_scale": 1.0},
    ("layer4", "k_down"): {"source_sha256_prefix": "5271af809b8e5ad3", "fetch_kib": 5929.5, "write_kib": 16.0,
                           "fetch_scale": 2.0, "write_scale": 1.0},
    ("batch32", "k_grouped_gateup"): {"source_sha256_prefix": "8bcffc6967ec026c", "fetch_kib": 576830.0,
                                      "write_kib": 3622.5, "fetch_scale": 2.0, "write_scale": 1.0},
    ("batch32", "k_grouped_down"): {"source_sha256_prefix": "8bcffc6967ec026c", "fetch_kib": 289846.8,
                                    "write_kib": 6145.0, "fetch_scale": 2.0, "write_scale": 1.0},
}


def kernel_source_hash(grouped):
    """sha256 of the sources the expert kernels are built from."""
    h = hashlib.sha256()
    names = ["moe_device.h", "moe_internal.h", "moe_layout.h",
             "moe_grouped.hip" if grouped else "moe_forward.hip"]
    for n in names:
        with open(os.path.join(ROOT, "bit_dequant_expert_router_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2048)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--workload", default="layer4", choices=["layer4", "layer2", "batch32", "tiny", "tier4"])
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
    p.add_argument("--quiet", action="store_true")
    return p.parse_args()


def log(args, msg):
    if not args.quiet:
        print(msg, file=sys.stderr, flush=True)


def main():
    args = parse_args()
    if args.gpus != 1:
        msg = (f"bench.py: --gpus {args.gpus} is not supported: this build runs the expert layer on one GPU "
               "(every expert resident in that GPU's HBM); run with --gpus 1")
        print(msg, flush=True)
        print(msg, file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_dequant_expert_router_amd as moe
    import synthetic as syn
    from bit_dequant_expert_router_amd.weights import layer_generated

    wl = syn.WORKLOADS[args.workload]
    if wl.name == "tier4":
        return bench_tier(args, wl)
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
    ridx = torch.empty((P, T, K), dtype=torch.int32, device=dev)
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

    # warmup
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region
    nsteps = args.steps
    graph = None
    if args.mode == "graph":
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                for i in range(nsteps):
                    step(i)
        torch.cuda.synchronize()
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
    ms_per_step = elapsed * 1e3 / nsteps
    tokens_per_s = nsteps * T / elapsed

    # algorithmic expert-weight bytes: distinct selected experts per step + shared
    idx_all = ridx.cpu().numpy()
    eb = moe.moe_expert_bytes(dims)
    distinct = [len(np.unique(idx_all[j].ravel())) + 1 for j in range(P)]
    steps_idx = [i % P for i in range(nsteps)]
    bytes_total = float(sum(distinct[j] for j in steps_idx)) * eb
    bytes_per_step = bytes_total / nsteps
    router_bytes = dims.n_experts * dims.hidden * 2

    # per-kernel durations, marginal: NW steps (token j, layer j mod R) get a
    # workspace each, filled by one full forward; for each stage s a HIP graph
    # of M steps running stages 0..s is replayed between two events on the
    # launch stream, and stage s is charged (elapsed(0..s) - elapsed(0..s-1)) / M
    NW = min(P, 64)
    wss = [torch.empty(wsb, dtype=torch.uint8, device=dev) for _ in range(NW)]
    for w in wss:
        moe.moe_workspace_init(w)
    for j in range(NW):
        moe.moe_layer_forward(dims, descs[j % R], pool[j], out[j], T, ridx[j], rw[j], wss[j], wsb)
    torch.cuda.synchronize()
    n_stages = moe.moe_forward_stage_count(dims, T)
    grouped = n_stages == 7
    if grouped:
        names = ["k_norm_batch", "k_router_mfma", "k_route_tokens", "k_grouped_gateup", "k_encode_act",
                 "k_grouped_down", "k_combine"]
        gu_stage, down_stage = 3, 5
        M = 64
    else:
        names = ["k_router", "k_gateup", "k_down"]
        gu_stage, down_stage = 1, 2
        M = 512
    prefix_s = []
    for last in range(n_stages):
        sg = torch.cuda.Stream()
        sg.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(sg):
            with torch.cuda.graph(g, stream=sg):
                for i in range(M):
                    j = i % NW
                    for st in range(last + 1):
                        moe.moe_layer_forward_stage(dims, descs[j % R], pool[j], out[j], T, ridx[j], rw[j], wss[j],
                                                    wsb, st)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        best = None
        for _ in range(2):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            # replay() launches the graph on the current stream: the events bracket it there
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            el = e0.elapsed_time(e1) * 1e-3 / M
            best = el if best is None else min(best, el)
        prefix_s.append(best)
        del g
    stage_s = np.diff(np.array([0.0] + prefix_s))
    stage_mean = np.array(stage_s)
    # algorithmic bytes of the expert kernels: gate + up (or down) codes and
    # scale/bias of the distinct selected experts and the shared one
    per_matrix = dims.ffn * dims.hidden * dims.bits // 8 + (dims.ffn * dims.hidden // 64) * 4
    n_distinct = float(np.mean([distinct[j] for j in range(NW)]))
    kbytes = {gu_stage: n_distinct * 2 * per_matrix, down_stage: n_distinct * per_matrix}
    dom = max(kbytes, key=lambda k: stage_mean[k])
    achieved = kbytes[dom] / stage_mean[dom]
    traffic = None
    tr = KERNEL_TRAFFIC.get((wl.name, names[dom])) if T == wl.n_tokens else None
    if tr is not None and tr["source_sha256_prefix"] == kernel_source_hash(grouped)[:16]:
        traffic = round((tr["fetch_kib"] * tr["fetch_scale"] + tr["write_kib"] * tr["write_scale"]) * 1024)

    result = {
        "metric": "MoE-layer decode tokens/s (effective expert-weight HBM GB/s and % of peak alongside)",
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
        "roofline": {
            "kernel": names[dom],
            "bound": "hbm",
            "achieved": round(achieved / 1e9, 1),
            "peak": HBM_PEAK_BPS / 1e9,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_BPS, 4),
            "traffic": traffic,
            "bytes_per_launch": round(kbytes[dom]),
            "launch_us": round(float(stage_mean[dom]) * 1e6, 3),
        },
        "stage_us": {n: round(float(v) * 1e6, 3) for n, v in zip(names, stage_mean)},
    }

    if args.cpu_sample > 0:
        result["cpu_baseline"] = cpu_baseline(args, wl, dims)

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
        "metric": "MoE-layer decode tokens/s (effective expert-weight HBM GB/s and % of peak alongside)",
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


def cpu_baseline(args, wl, dims):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np

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


if __name__ == "__main__":
    main()
