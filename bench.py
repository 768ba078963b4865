"""Benchmark of the routed MoE layer on one MI355X.

Workload (default): the gpt-oss-120B-shaped decode layer, T = 1 token, H = 2880,
I = 2880, E = 128 experts, top-4, MXFP4 experts (13,219,200 B each), bf16
activations, router bias ~ N(0, 0.5).  One step = one whole layer forward (router,
top-k, bucketing, fused gate/up + SwiGLU, down, combine) on one token.

Steps rotate over a bank of independently seeded layer instances resident in HBM,
each with its own input token, so that a step's experts were last touched several
hundred MB of traffic earlier and are read from HBM rather than from the 256 MB
Infinity Cache.

Prints one JSON line.  `roofline` covers the dominant kernel (the fused gate/up +
SwiGLU, about 2/3 of the layer's bytes): algorithmic bytes per launch (the packed
gate/up matrices of the distinct selected experts plus the activations) over the
kernel's average execution time, stamped by the kernel's dispatch packet on its own
stream during the timed steps.  `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode), TFLOP/s (prefill), 1 GPU"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_c2_gateup.json")
KERNEL_SOURCES = ["quantized_mixture_experts_amd/csrc/k_experts.hip", "quantized_mixture_experts_amd/csrc/device.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", default="c2", choices=["c1", "c2", "c3", "c5a", "c5b"])
    ap.add_argument("--layers", type=int, default=None, help="distinct layer instances in the rotation")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU-oracle sample budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    return ap.parse_args()


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only: this layer is built and measured on a single MI355X "
              f"(--gpus {args.gpus} requested); multi-GPU sharding is a design note, not a run.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import quantized_mixture_experts_amd as q
    import synth

    q.lib()
    dev = torch.device("cuda:0")
    spec = synth.CONFIGS[args.config]
    T, H, I, E, k = spec.T, spec.hidden, spec.inter, spec.n_experts, spec.top_k
    nl = args.layers or {"c1": 4, "c2": 16, "c3": 16, "c5a": 4, "c5b": 4}[args.config]

    # ---- resident bank of layer instances -------------------------------------
    t0 = time.time()
    layers, xs = [], []
    for l in range(nl):
        host = synth.make_layer(spec, layer=l)
        layers.append(q.DeviceLayer.from_layer(host, device=dev))
        del host
        xs.append(torch.from_numpy(synth.make_x(spec, layer=l)).to(dev))
        log(args, f"layer instance {l + 1}/{nl} resident ({time.time() - t0:.1f} s)")
    ws = layers[0].workspace(T)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)

    # routing of each instance (for the algorithmic byte count: distinct experts)
    distinct = []
    for l in range(nl):
        _, dbg = q.forward(layers[l], xs[l], spec.x_dtype, y=y, ws=ws, debug=True)
        distinct.append(len(np.unique(dbg["ids"].cpu().numpy())))
    torch.cuda.synchronize()

    gu_bytes = q.packed_bytes(spec.weights.wfmt, 2 * I, H)
    dn_bytes = q.packed_bytes(spec.weights.wfmt, H, I)
    xb = 4 if spec.x_dtype == synth.X_F32 else 2
    sh = spec.has_shared

    def step_bytes(l):
        d = distinct[l] + sh
        router = E * H * 4 + (E * 4 if spec.bias != "none" else 0)
        return d * (gu_bytes + dn_bytes) + router + T * H * xb + T * H * 4

    def gateup_bytes(l):
        return (distinct[l] + sh) * gu_bytes + T * H * xb

    def step_flops():
        P = T * k + T * sh
        return 2 * T * E * H + P * 6 * H * I

    # ---- the timed region: HIP-graph replays of whole steps --------------------------
    # One graph holds one step per layer instance (nl steps); K steps = K / nl replays.
    K, W = args.steps, args.warmup
    K = max(nl, (K // nl) * nl)
    NS = len(q.STAGES)
    for s in range(W):
        l = s % nl
        q.forward(layers[l], xs[l], spec.x_dtype, y=y, ws=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for l in range(nl):
            q.forward(layers[l], xs[l], spec.x_dtype, y=y, ws=ws)
    for _ in range(max(1, W // nl)):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K // nl):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    ms_per_step = total_ms / K

    # ---- kernel durations: the same K steps launched eagerly, each kernel carrying its
    # own start/stop events (stamped by its dispatch packet on the layer's stream) -------
    events = q.HipEvents(2 * NS * K)
    ee0, ee1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ee0.record()
    for s in range(K):
        l = s % nl
        q.forward_timed(layers[l], xs[l], spec.x_dtype, y, ws, events.slice(2 * NS * s, 2 * NS))
    ee1.record()
    torch.cuda.synchronize()
    eager_ms_per_step = ee0.elapsed_time(ee1) / K

    stage_ms = {}
    for st, name in enumerate(q.STAGES):
        vals = [events.elapsed_ms(2 * NS * s + 2 * st, 2 * NS * s + 2 * st + 1) for s in range(K)]
        vals = [v for v in vals if v is not None]
        if vals:
            stage_ms[name] = sum(vals) / len(vals)
    gu_ms = stage_ms.get("gateup")
    gu_b = sum(gateup_bytes(s % nl) for s in range(K)) / K
    achieved = gu_b / (gu_ms * 1e-3) / 1e9 if gu_ms else None
    sb = sum(step_bytes(s % nl) for s in range(K)) / K
    tokens_per_s = T * K / (total_ms * 1e-3)

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        if tr.get("kernel_source_hash") == kernel_source_hash():
            traffic = tr.get("bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.config}: {spec.name}, T={T}, H={H}, I={I}, E={E}"
                        f"{'+1 shared' if sh else ''}, top-{k}, "
                        f"{'MXFP4' if spec.weights.wfmt == synth.WFMT_MXFP4 else '4-bit codebook'} experts",
            "layer_instances_rotated": nl,
            "global_batch": T,
        },
        "timing": "HIP-graph replay of whole steps; kernel durations from an eager pass of the same steps",
        "eager_ms_per_step": round(eager_ms_per_step, 6),
        "layer_hbm_gbs": round(sb / (ms_per_step * 1e-3) / 1e9, 1),
        "layer_bytes_per_step": int(sb),
        "layer_tflops": round(step_flops() / (ms_per_step * 1e-3) / 1e12, 3),
        "stage_us": {n: round(v * 1e3, 2) for n, v in stage_ms.items()},
        "roofline": {
            "kernel": "gateup (fused dequant + gate/up + SwiGLU)",
            "bound": "hbm",
            "achieved": round(achieved, 1) if achieved else None,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4) if achieved else None,
            "traffic": traffic,
            "bytes_per_launch": int(gu_b),
            "avg_us": round(gu_ms * 1e3, 2) if gu_ms else None,
        },
        "cpu_baseline": None,
    }

    # ---- CPU oracle on a bounded sample -------------------------------------------
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, spec, nl)

    print(json.dumps(result), flush=True)


def cpu_baseline(args, spec, nl):
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = 1
    spent, tokens, layers_used = 0.0, 0, 0
    for l in range(max(nl, 64)):
        x = synth.make_x(spec, layer=l)
        router_only = synth.make_layer(spec, layer=l, experts=[])
        x64 = oracle.activations_f64(x, spec.x_dtype)
        ids, _ = oracle.topk_softmax(oracle.router_logits(x64, router_only.router_w, router_only.router_b),
                                     spec.top_k)
        layer = synth.make_layer(spec, layer=l, experts=np.unique(ids))
        t0 = time.perf_counter()
        oracle.moe_forward(layer, x, spec.x_dtype)
        spent += time.perf_counter() - t0
        tokens += x.shape[0]
        layers_used += 1
        log(args, f"cpu oracle: {tokens} tokens in {spent:.1f} s")
        if spent >= args.cpu_seconds:
            break
    return {"value": round(tokens / spent, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{tokens} tokens of the same workload ({layers_used} seeded layer instances, "
                      f"each token through its own layer), fp64 numpy oracle, {spent:.1f} s of oracle time"}


if __name__ == "__main__":
    main()
