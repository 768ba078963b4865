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
RMS_EPS = 1e-6  # eps of the RMS rescale between the stacked layers
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_c2_gateup.json")
CSRC = os.path.join(ROOT, "quantized_mixture_experts_amd", "csrc")


def kernel_source_hash() -> str:
    """Hash of every kernel source: stored counter readings are used only while it matches."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        h.update(name.encode())
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", default="c2", choices=["c1", "c2", "c3", "c4", "c5a", "c5b"])
    ap.add_argument("--tokens", type=int, default=None, help="override T (the stacked config runs T=1 and T=4; "
                    "the verify config with T=136 is the batched verify round of 8 requests x 17 tokens)")
    ap.add_argument("--path", choices=["auto", "decode", "prefill"], default="auto",
                    help="kernel path (auto: decode kernels up to 32 tokens)")
    ap.add_argument("--layers", type=int, default=None, help="distinct layer instances in the rotation")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU-oracle sample budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="eager steps only (no graph), then a plain 1 GiB device copy that calibrates the "
                         "HBM byte counters; meant to run under rocprofv3 --pmc")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 counter CSVs of a --counters run into the stored "
                         "per-launch HBM traffic of the gate/up kernel")
    ap.add_argument("--quiet", action="store_true")
    return ap.parse_args()


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


COPY_BYTES = 1 << 30


class Workload:
    """Resident layer instances and inputs of one config, and what one step enqueues."""

    def __init__(self, args, spec, dev):
        import torch
        import quantized_mixture_experts_amd as q
        import synth
        self.q, self.spec = q, spec
        self.T = args.tokens or spec.T
        self.path = {"auto": q.PATH_AUTO, "decode": q.PATH_DECODE, "prefill": q.PATH_PREFILL}[args.path]
        self.stacked = spec.n_layers > 1
        if self.stacked:
            nl = spec.n_layers
        else:
            nl = args.layers or {"c1": 4, "c2": 16, "c3": 16, "c5a": 4, "c5b": 4}[args.config]
        self.nl = nl
        t0 = time.time()
        self.layers, self.xs = [], []
        for l in range(nl):
            host = synth.make_layer(spec, layer=l)
            self.layers.append(q.DeviceLayer.from_layer(host, device=dev))
            del host
            self.xs.append(torch.from_numpy(synth.make_x(spec, T=self.T, layer=l)).to(dev))
            log(args, f"layer instance {l + 1}/{nl} resident ({time.time() - t0:.1f} s)")
        self.ws = self.layers[0].workspace(self.T)
        H = spec.hidden
        # stacked: y_l feeds x_{l+1} through the RMS rescale; single layers share one y
        self.ys = [torch.empty((self.T, H), dtype=torch.float32, device=dev)
                   for _ in range(nl if self.stacked else 1)]
        self.forwards_per_step = nl if self.stacked else 1
        self.steps_per_graph = 1 if self.stacked else nl

    def _chain(self, s, fn, fn_rms=None):
        """Enqueue step s; fn(layer_index, x, y) enqueues one layer forward.  Stacked:
        layer l > 0 takes the RMS rescale of y_{l-1}, through fn_rms(l, y_prev, y) (the
        rescale inside the layer call) when given, else as a separate rescale and fn."""
        q = self.q
        if self.stacked:
            fn(0, self.xs[0], self.ys[0])
            for l in range(1, self.nl):
                if fn_rms is not None:
                    fn_rms(l, self.ys[l - 1], self.ys[l])
                else:
                    q.rms_rescale(self.ys[l - 1], out=self.xs[l])
                    fn(l, self.xs[l], self.ys[l])
        else:
            l = s % self.nl
            fn(l, self.xs[l], self.ys[0])

    def step(self, s):
        q, xd = self.q, self.spec.x_dtype
        self._chain(s, lambda l, x, y: q.forward(self.layers[l], x, xd, y=y, ws=self.ws, path=self.path),
                    lambda l, yp, y: q.forward_rms(self.layers[l], yp, RMS_EPS, y=y, ws=self.ws, path=self.path))

    def step_timed(self, s, events, ev0):
        q, xd, NS = self.q, self.spec.x_dtype, len(self.q.STAGES)
        ctr = [ev0]

        def fn(l, x, y):
            q.forward_timed(self.layers[l], x, xd, y, self.ws, events.slice(ctr[0], 2 * NS), path=self.path)
            ctr[0] += 2 * NS

        def fn_rms(l, yp, y):
            q.forward_rms(self.layers[l], yp, RMS_EPS, y=y, ws=self.ws, events=events.slice(ctr[0], 2 * NS),
                          path=self.path)
            ctr[0] += 2 * NS
        self._chain(s, fn, fn_rms)

    def distinct_experts(self):
        """Distinct routed experts of every forward of one rotation (for the byte counts)."""
        import numpy as np
        out = []
        for s in range(self.steps_per_graph):
            def fn(l, x, y):
                _, dbg = self.q.forward(self.layers[l], x, self.spec.x_dtype, y=y, ws=self.ws, debug=True)
                out.append(len(np.unique(dbg["ids"].cpu().numpy())))
            self._chain(s, fn)
        return out


def main():
    args = parse()
    if args.traffic_from:
        write_traffic(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only: this layer is built and measured on a single MI355X "
              f"(--gpus {args.gpus} requested); multi-GPU sharding is a design note, not a run.", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_mixture_experts_amd as q
    import synth

    q.lib()
    dev = torch.device("cuda:0")
    spec = synth.CONFIGS[args.config]
    wl = Workload(args, spec, dev)
    T, H, I, E, k = wl.T, spec.hidden, spec.inter, spec.n_experts, spec.top_k
    sh = spec.has_shared
    distinct = wl.distinct_experts()  # one entry per forward of a rotation
    torch.cuda.synchronize()

    if args.counters:
        for s in range(max(args.steps, 1)):
            wl.step(s)
        torch.cuda.synchronize()
        a = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"counters_run": args.config, "steps": args.steps, "copy_bytes": COPY_BYTES,
                          "gateup_bytes_per_launch": gateup_bytes_avg(spec, T, distinct),
                          "kernel_source_hash": kernel_source_hash()}), flush=True)
        return

    gu_bytes = q.packed_bytes(spec.weights.wfmt, 2 * I, H)
    dn_bytes = q.packed_bytes(spec.weights.wfmt, H, I)
    xb = 4 if spec.x_dtype == synth.X_F32 else 2

    def fwd_bytes(d):
        router = E * H * 4 + (E * 4 if spec.bias != "none" else 0)
        return (d + sh) * (gu_bytes + dn_bytes) + router + T * H * xb + T * H * 4

    def fwd_flops():
        P = T * k + T * sh
        return 2 * T * E * H + P * 6 * H * I

    # ---- the timed region: HIP-graph replays of whole steps --------------------------
    K, W = args.steps, args.warmup
    spg = wl.steps_per_graph
    K = max(spg, (K // spg) * spg)
    NS = len(q.STAGES)
    for s in range(W):
        wl.step(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(spg):
            wl.step(s)
    for _ in range(max(1, W // spg)):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K // spg):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    ms_per_step = total_ms / K

    # ---- kernel durations: the same K steps launched eagerly, each kernel carrying its
    # own start/stop events (stamped by its dispatch packet on the layer's stream) -------
    fps = wl.forwards_per_step
    events = q.HipEvents(2 * NS * fps * K)
    ee0, ee1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ee0.record()
    for s in range(K):
        wl.step_timed(s, events, 2 * NS * fps * s)
    ee1.record()
    torch.cuda.synchronize()
    eager_ms_per_step = ee0.elapsed_time(ee1) / K

    # per-forward stage durations; forward f of step s is rotation entry (s % spg) * fps + f
    stage_ms, moe_ms_per_step = {}, 0.0
    for st, name in enumerate(q.STAGES):
        vals = []
        for s in range(K):
            for f in range(fps):
                b = 2 * NS * (fps * s + f) + 2 * st
                v = events.elapsed_ms(b, b + 1)
                if v is not None:
                    vals.append(v)
        if vals:
            stage_ms[name] = sum(vals) / len(vals)
            moe_ms_per_step += stage_ms[name] * fps
    gu_ms = stage_ms.get("gateup")
    gu_b = gateup_bytes_avg(spec, T, distinct)
    achieved = gu_b / (gu_ms * 1e-3) / 1e9 if gu_ms else None
    sb = sum(fwd_bytes(d) for d in distinct) / len(distinct) * fps
    tokens_per_s = T * K / (total_ms * 1e-3)

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        if tr.get("kernel_source_hash") == kernel_source_hash() and tr.get("config") == args.config:
            traffic = tr.get("bytes_per_launch")

    fmt = "MXFP4" if spec.weights.wfmt == synth.WFMT_MXFP4 else "4-bit codebook"
    workload = (f"{args.config}: {spec.name}, T={T}, H={H}, I={I}, E={E}{'+1 shared' if sh else ''}, "
                f"top-{k}, {fmt} experts" + (f", {spec.n_layers} stacked layers" if wl.stacked else "")
                + (f", {args.path} kernels forced" if args.path != "auto" else ""))
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
            "workload": workload,
            "layer_instances": wl.nl,
            "global_batch": T,
        },
        "timing": "HIP-graph replay of whole steps; kernel durations from an eager pass of the same steps",
        "eager_ms_per_step": round(eager_ms_per_step, 6),
        "moe_kernels_ms_per_step": round(moe_ms_per_step, 6),
        "layer_hbm_gbs": round(sb / (ms_per_step * 1e-3) / 1e9, 1),
        "algorithmic_bytes_per_step": int(sb),
        "tflops": round(fwd_flops() * fps / (ms_per_step * 1e-3) / 1e12, 3),
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
        result["cpu_baseline"] = cpu_baseline(args, spec, T, wl.nl, wl.stacked)

    print(json.dumps(result), flush=True)


def gateup_bytes_avg(spec, T, distinct):
    """Algorithmic bytes of one gate/up launch: the packed gate/up matrices of the distinct
    selected experts (plus the shared one) and the activations, averaged over launches."""
    import quantized_mixture_experts_amd as q
    import synth
    gu = q.packed_bytes(spec.weights.wfmt, 2 * spec.inter, spec.hidden)
    xb = 4 if spec.x_dtype == synth.X_F32 else 2
    return sum((d + spec.has_shared) * gu + T * spec.hidden * xb for d in distinct) / len(distinct)


def _counter_rows(path):
    import csv
    with open(path) as f:
        for row in csv.DictReader(f):
            yield row


def _per_kernel(path, counter):
    """{kernel name: [value per dispatch]} for one counter of a rocprofv3 counter CSV."""
    out = {}
    for row in _counter_rows(path):
        if row.get("Counter_Name") != counter:
            continue
        out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def write_traffic(args):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the gate/up kernel, each scaled by
    what the same counter reads for the 1 GiB plain copy of the same run."""
    fetch = _per_kernel(args.traffic_from[0], "FETCH_SIZE")
    write = _per_kernel(args.traffic_from[1], "WRITE_SIZE")

    def copy_kib(d):
        # torch's same-dtype device copy is a runtime blit; the calibration copies are the
        # three largest of its dispatches (the others are the small uploads of the set-up)
        name = next((n for n in d if "copyBuffer" in n), None)
        if name is None:
            raise SystemExit("no device copy kernel in the counter CSV")
        top = sorted(d[name])[-3:]
        return sum(top) / len(top), name

    fcopy, fname = copy_kib(fetch)
    wcopy, _ = copy_kib(write)
    f_scale = COPY_BYTES / (fcopy * 1024.0)
    w_scale = COPY_BYTES / (wcopy * 1024.0)
    gu = [n for n in fetch if "gateup" in n]
    if not gu:
        raise SystemExit("no gate/up kernel in the counter CSV")
    per_kernel = {}
    for n in gu:
        fv, wv = fetch[n], write.get(n, [0.0])
        per_kernel[n] = {"launches": len(fv), "fetch_kib_avg": sum(fv) / len(fv), "write_kib_avg": sum(wv) / len(wv)}
    # the launch-weighted mean over every gate/up instantiation that ran
    nlaunch = sum(v["launches"] for v in per_kernel.values())
    fb = sum(v["fetch_kib_avg"] * v["launches"] for v in per_kernel.values()) / nlaunch * 1024.0 * f_scale
    wb = sum(v["write_kib_avg"] * v["launches"] for v in per_kernel.values()) / nlaunch * 1024.0 * w_scale
    meta = {}
    meta_path = os.path.join(os.path.dirname(os.path.abspath(args.traffic_from[0])), "counters_run.json")
    if os.path.exists(meta_path):
        meta = json.load(open(meta_path))
    out = {
        "config": meta.get("counters_run", "c2"),
        "kernel_source_hash": meta["kernel_source_hash"] if "kernel_source_hash" in meta else kernel_source_hash(),
        "bytes_per_launch": int(round(fb + wb)),
        "fetch_bytes_per_launch": int(round(fb)),
        "write_bytes_per_launch": int(round(wb)),
        "algorithmic_bytes_per_launch": meta.get("gateup_bytes_per_launch"),
        "calibration": {"copy_kernel": fname, "copy_bytes": COPY_BYTES, "fetch_kib": fcopy, "write_kib": wcopy,
                        "fetch_scale": f_scale, "write_scale": w_scale},
        "kernels": per_kernel,
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def cpu_baseline(args, spec, T, nl, stacked):
    """The oracle as it stands, on a bounded sample of the same workload: whole layers of
    independently seeded instances (each with its own input rows) until the time budget
    is spent.  For the stacked config one token's step is 36 layers, so the rate is the
    sampled per-layer time times the depth."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = 1
    spent, layers_used = 0.0, 0
    for l in range(max(nl, 64)):
        x = synth.make_x(spec, T=T, layer=l)
        router_only = synth.make_layer(spec, layer=l, experts=[])
        x64 = oracle.activations_f64(x, spec.x_dtype)
        ids, _ = oracle.topk_softmax(oracle.router_logits(x64, router_only.router_w, router_only.router_b),
                                     spec.top_k)
        layer = synth.make_layer(spec, layer=l, experts=np.unique(ids))
        t0 = time.perf_counter()
        oracle.moe_forward(layer, x, spec.x_dtype)
        spent += time.perf_counter() - t0
        layers_used += 1
        log(args, f"cpu oracle: {layers_used} layer forwards of {T} tokens in {spent:.1f} s")
        if spent >= args.cpu_seconds:
            break
    depth = spec.n_layers if stacked else 1
    tokens_per_s = T * layers_used / spent / depth
    what = (f"{layers_used} forwards of {T} token(s) through seeded instances of the layer"
            + (f", scaled by the {depth}-layer depth" if stacked else "")
            + f"; fp64 numpy oracle, {spent:.1f} s of oracle time")
    return {"value": round(tokens_per_s, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": what}


if __name__ == "__main__":
    main()
