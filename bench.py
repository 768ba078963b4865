"""Benchmark of the routed MoE layer on one MI355X.

Workload (default): 36 stacked gpt-oss-120B-shaped MoE layers (H = 2880, I = 2880,
E = 128 experts, top-4, MXFP4 experts of 13,219,200 B, about 61 GB of experts resident
in HBM), bf16 activations, router bias ~ N(0, 0.5).  One step = one token batch through
all 36 layers: layer 0 takes x, every later layer takes the fp64 RMS rescale of the
previous layer's fp32 output (inside the layer call).  T = 1 gives `value`; T = 4 is
reported beside it.  Every layer's experts are distinct, so each step reads its experts
from HBM (1.96 GB per token at T = 1), not from the 256 MB Infinity Cache.

Other workloads (--config): the single decode layer (c2), the verify window (c3), the
tiny layer (c1) and the two 1,024-token prefill chunks (c5a, c5b).  Single-layer steps
rotate over several independently seeded layer instances resident in HBM for the same
reason.

Prints one JSON line.  `roofline` covers the dominant kernel (the fused gate/up +
SwiGLU, about 2/3 of the layer's bytes): algorithmic bytes per launch (the packed gate/up
matrices of the distinct selected experts plus the activations) over the kernel's
average execution time, stamped by its dispatch packet on its own stream.
`step_roofline` is the whole step's algorithmic bytes over the step time.  Every
fraction is also given against the streaming-read probe's measured bandwidth.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
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
BF16_PEAK_TFLOPS = 2500.0
RMS_EPS = 1e-6  # eps of the RMS rescale between the stacked layers (passed as fp32)
CSRC = os.path.join(ROOT, "quantized_mixture_experts_amd", "csrc")
PROBE_BYTES = 4 << 30
PROBE_BLOCKS = 4096


def traffic_file(config: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{config}_gateup.json")


def strip_comments(src: str) -> str:
    """C/C++ source without its comments and blank lines (string and character literals kept)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return "\n".join(ln.rstrip() for ln in "".join(out).splitlines() if ln.strip())


def kernel_source_hash() -> str:
    """Hash of every kernel source with its comments removed: stored counter readings are used
    only while it matches, so an edit of a comment keeps them and any code change drops them."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        h.update(name.encode())
        h.update(strip_comments(open(os.path.join(CSRC, name), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c4", choices=["c1", "c2", "c3", "c4", "c5a", "c5b", "aff3"])
    ap.add_argument("--tokens", type=int, default=None, help="override T (the stacked config runs T=1 and T=4; "
                    "the verify config with T=136 is the batched verify round of 8 requests x 17 tokens)")
    ap.add_argument("--path", choices=["auto", "decode", "prefill"], default="auto",
                    help="kernel path (auto: decode kernels for small batches)")
    ap.add_argument("--layers", type=int, default=None, help="distinct layer instances in the rotation")
    ap.add_argument("--omit", type=float, default=0.0,
                    help="marginal-expert omission threshold (routed pairs with a gate below it are left out; "
                         "0: off)")
    ap.add_argument("--packed-scales", action="store_true",
                    help="MXFP4 workloads: the same experts in the packed scale store (a base E8M0 byte per row "
                         "and a 4-bit delta per block)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU-oracle sample budget (wall)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="eager steps only (no graph), then a plain 1 GiB device copy that calibrates the "
                         "HBM byte counters; meant to run under rocprofv3 --pmc")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 counter CSVs of a --counters run into the stored "
                         "per-launch HBM traffic of the gate/up kernel")
    ap.add_argument("--traffic-kernel", default="k_dec_gateup",
                    help="substring of the kernel name whose counters --traffic-from averages")
    ap.add_argument("--quiet", action="store_true")
    return ap.parse_args()


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


COPY_BYTES = 1 << 30


class Workload:
    """Resident layer instances of one config, and what one step enqueues for T tokens."""

    def __init__(self, args, spec, dev):
        import quantized_mixture_experts_amd as q
        import synth
        self.q, self.spec, self.dev = q, spec, dev
        self.path = {"auto": q.PATH_AUTO, "decode": q.PATH_DECODE, "prefill": q.PATH_PREFILL}[args.path]
        self.stacked = spec.n_layers > 1
        if self.stacked:
            nl = spec.n_layers
        else:
            nl = args.layers or {"c1": 4, "c2": 16, "c3": 16, "c5a": 4, "c5b": 4, "aff3": 16}[args.config]
        self.nl = nl
        t0 = time.time()
        self.layers = []
        for l in range(nl):
            host = synth.make_layer(spec, layer=l)
            self.layers.append(q.DeviceLayer.from_layer(host, device=dev, omit_below=args.omit))
            del host
            log(args, f"layer instance {l + 1}/{nl} resident ({time.time() - t0:.1f} s)")
        self.forwards_per_step = nl if self.stacked else 1
        self.set_tokens(spec.T)

    def set_tokens(self, T):
        import torch
        import synth
        self.T = T
        self.xs = [torch.from_numpy(synth.make_x(self.spec, T=T, layer=l)).to(self.dev)
                   for l in range(1 if self.stacked else self.nl)]
        self.ws = self.layers[0].workspace(T)
        H = self.spec.hidden
        # stacked: y_l feeds layer l+1 through the RMS rescale; single layers share one y
        self.ys = [torch.empty((T, H), dtype=torch.float32, device=self.dev)
                   for _ in range(self.nl if self.stacked else 1)]

    def rotation(self):
        """Steps after which the inputs repeat: one (stacked) or one per layer instance."""
        return 1 if self.stacked else self.nl

    def _chain(self, s, fn, fn_rms):
        """Enqueue step s: fn(l, x, y) enqueues a layer forward on x, fn_rms(l, y_prev, y)
        one on the RMS rescale of y_prev (stacked layers 1..)."""
        if self.stacked:
            fn(0, self.xs[0], self.ys[0])
            for l in range(1, self.nl):
                fn_rms(l, self.ys[l - 1], self.ys[l])
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
        for s in range(self.rotation()):
            def fn(l, x, y):
                _, dbg = self.q.forward(self.layers[l], x, self.spec.x_dtype, y=y, ws=self.ws, debug=True)
                ids = dbg["ids"].cpu().numpy()
                out.append(len(np.unique(ids[ids >= 0])))  # -1: an omitted pair

            def fn_rms(l, yp, y):
                xr = self.q.rms_rescale(yp, RMS_EPS)
                fn(l, xr, y)
            self._chain(s, fn, fn_rms)
        return out


def pct(vals, p):
    v = sorted(vals)
    i = min(len(v) - 1, max(0, int(round(p / 100.0 * (len(v) - 1)))))
    return v[i]


def measure(args, wl, T, probe_gbs):
    """Graph-replayed timing of K steps at T tokens, then the per-kernel durations of an
    eager pass of the same K steps."""
    import torch
    import quantized_mixture_experts_amd as q
    import synth
    spec = wl.spec
    wl.set_tokens(T)
    H, I, E, k, sh = spec.hidden, spec.inter, spec.n_experts, spec.top_k, spec.has_shared
    distinct = wl.distinct_experts()  # one entry per forward of a rotation
    torch.cuda.synchronize()
    gu_bytes = q.packed_bytes(spec.weights.wfmt, 2 * I, H)
    dn_bytes = q.packed_bytes(spec.weights.wfmt, H, I)
    xb = 4 if spec.x_dtype == synth.X_F32 else 2

    def fwd_bytes(d):
        router = E * H * 4 + (E * 4 if spec.bias != "none" else 0)
        return (d + sh) * (gu_bytes + dn_bytes) + router + T * H * xb + T * H * 4

    P = T * k + T * sh
    fwd_flops = 2 * T * E * H + P * 6 * H * I

    K, W = args.steps, args.warmup
    for s in range(W):
        wl.step(s)
    torch.cuda.synchronize()
    # one graph per chunk of steps: the stacked config's step is 108 kernels (a graph per
    # step); single-layer steps are a few kernels, so a graph holds the whole rotation over
    # the layer instances (plus a graph of the remaining steps, so exactly K steps run)
    per = 1 if wl.stacked else wl.nl
    chunks = [per] * (K // per) + ([K % per] if K % per else [])

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(n):
                wl.step(s)
        return g
    graphs = {n: capture(n) for n in sorted(set(chunks))}
    for _ in range(max(1, W // per)):
        graphs[per].replay()
    torch.cuda.synchronize()
    # ---- the timed region: K graph-replayed steps, an event between consecutive chunks ----
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(chunks) + 1)]
    evs[0].record()
    for i, n in enumerate(chunks):
        graphs[n].replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    total_ms = evs[0].elapsed_time(evs[-1])
    step_ms = [evs[i].elapsed_time(evs[i + 1]) / n for i, n in enumerate(chunks)]
    ms_per_step = total_ms / K
    del graphs

    # ---- kernel durations: the same K steps launched eagerly, each kernel carrying its own
    # start/stop events (stamped by its dispatch packet on the layer's stream) ----
    NS = len(q.STAGES)
    fps = wl.forwards_per_step
    events = q.HipEvents(2 * NS * fps * K)
    ee0, ee1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ee0.record()
    for s in range(K):
        wl.step_timed(s, events, 2 * NS * fps * s)
    ee1.record()
    torch.cuda.synchronize()
    eager_ms_per_step = ee0.elapsed_time(ee1) / K
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
    del events

    gu_ms = stage_ms.get("gateup")
    gu_b = sum((d + sh) * gu_bytes + T * H * xb for d in distinct) / len(distinct)
    achieved = gu_b / (gu_ms * 1e-3) / 1e9 if gu_ms else None
    step_bytes = sum(fwd_bytes(d) for d in distinct) / len(distinct) * fps
    step_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    tokens_per_s = T * K / (total_ms * 1e-3)

    traffic = None
    tf = traffic_file(args.config)
    if os.path.exists(tf):
        tr = json.load(open(tf))
        if tr.get("kernel_source_hash") == kernel_source_hash() and tr.get("tokens") == T:
            traffic = tr.get("bytes_per_launch")

    def frac(a, p):
        return round(a / p, 4) if (a and p) else None

    return {
        "value": round(tokens_per_s, 2),
        "T": T,
        "ms_per_step": round(ms_per_step, 6),
        "step_ms_p10_p50_p90": [round(pct(step_ms, p), 6) for p in (10, 50, 90)],
        "eager_ms_per_step": round(eager_ms_per_step, 6),
        "moe_kernels_ms_per_step": round(moe_ms_per_step, 6),
        "moe_us_per_token": round(ms_per_step * 1e3 / T, 3),
        "hbm_gbs": round(step_gbs, 1),
        "tflops": round(fwd_flops * fps / (ms_per_step * 1e-3) / 1e12, 3),
        "algorithmic_bytes_per_step": int(step_bytes),
        "distinct_experts_per_forward": round(sum(distinct) / len(distinct), 2),
        "stage_us": {n: round(v * 1e3, 2) for n, v in stage_ms.items()},
        "roofline": {
            "kernel": "gateup (fused dequant + gate/up + SwiGLU)",
            "bound": "hbm",
            "achieved": round(achieved, 1) if achieved else None,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": frac(achieved, HBM_PEAK_GBS),
            "traffic": traffic,
            "bytes_per_launch": int(gu_b),
            "avg_us": round(gu_ms * 1e3, 2) if gu_ms else None,
            "probe_gbs": probe_gbs,
            "frac_of_probe": frac(achieved, probe_gbs),
        },
        "step_roofline": {
            "bound": "hbm",
            "achieved": round(step_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": frac(step_gbs, HBM_PEAK_GBS),
            "frac_of_probe": frac(step_gbs, probe_gbs),
            "roofline_us_per_step": round(step_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 3),
        },
    }


def hbm_probe(args, dev):
    """Streaming read of 4 GiB with 16-byte loads (the library's probe kernel): the best of
    five timed passes, GB/s."""
    import torch
    import quantized_mixture_experts_amd as q
    buf = torch.empty(PROBE_BYTES, dtype=torch.uint8, device=dev)
    buf.fill_(3)
    out = torch.empty(PROBE_BLOCKS, dtype=torch.int32, device=dev)
    q.hbm_read_probe(buf, out, PROBE_BLOCKS)
    torch.cuda.synchronize()
    best = None
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        q.hbm_read_probe(buf, out, PROBE_BLOCKS)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del buf, out
    torch.cuda.empty_cache()
    gbs = PROBE_BYTES / (best * 1e-3) / 1e9
    log(args, f"streaming-read probe: {gbs:.0f} GB/s")
    return round(gbs, 1)


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
    if args.packed_scales:
        spec = synth.with_packed_scales(spec)
    probe_gbs = None if (args.no_probe or args.counters) else hbm_probe(args, dev)
    wl = Workload(args, spec, dev)
    stacked = spec.n_layers > 1
    Ts = [args.tokens] if args.tokens else ([1, 4] if stacked else [spec.T])

    if args.counters:
        T = Ts[0]
        wl.set_tokens(T)
        distinct = wl.distinct_experts()
        for s in range(max(args.steps, 1)):
            wl.step(s)
        torch.cuda.synchronize()
        a = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        gu = q.packed_bytes(spec.weights.wfmt, 2 * spec.inter, spec.hidden)
        xb = 4 if spec.x_dtype == synth.X_F32 else 2
        gub = sum((d + spec.has_shared) * gu + T * spec.hidden * xb for d in distinct) / len(distinct)
        print(json.dumps({"counters_run": args.config, "tokens": T, "steps": args.steps, "copy_bytes": COPY_BYTES,
                          "gateup_bytes_per_launch": gub, "kernel_source_hash": kernel_source_hash()}), flush=True)
        return

    runs = []
    for T in Ts:
        r = measure(args, wl, T, probe_gbs)
        log(args, f"T={T}: {r['value']} tokens/s, {r['ms_per_step']} ms per step")
        runs.append(r)
    main_run = runs[0]

    fmt = {synth.WFMT_MXFP4: "MXFP4", synth.WFMT_CB4: "4-bit codebook",
           synth.WFMT_MXFP4_PS: "MXFP4 (packed scale store)",
           synth.WFMT_AFF3: "3-bit affine group-64"}[spec.weights.wfmt]
    H, I, E, k, sh = spec.hidden, spec.inter, spec.n_experts, spec.top_k, spec.has_shared
    workload = (f"{args.config}: {spec.name}, T={main_run['T']}, H={H}, I={I}, E={E}{'+1 shared' if sh else ''}, "
                f"top-{k}, {fmt} experts" + (f", {spec.n_layers} stacked layers (RMS rescale between)"
                                             if stacked else "")
                + (f", {args.path} kernels forced" if args.path != "auto" else "")
                + (f", marginal experts omitted below a gate of {args.omit}" if args.omit > 0 else ""))
    result = {
        "metric": METRIC,
        "value": main_run["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_run["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": workload,
            "layer_instances": wl.nl,
            "global_batch": main_run["T"],
        },
        "timing": "HIP-graph replay of whole steps (stacked: one graph per step; single layers: one graph "
                  "per rotation over the layer instances), an event between consecutive graphs; p10/p50/p90 "
                  "over graphs; kernel durations from an eager pass of the same steps with dispatch-stamped "
                  "events",
    }
    for key in ("step_ms_p10_p50_p90", "eager_ms_per_step", "moe_kernels_ms_per_step", "moe_us_per_token",
                "hbm_gbs", "tflops", "algorithmic_bytes_per_step", "distinct_experts_per_forward", "stage_us",
                "roofline", "step_roofline"):
        result[key] = main_run[key]
    if len(runs) > 1:
        result["other_batches"] = {f"T={r['T']}": r for r in runs[1:]}
    result["hbm_probe_gbs"] = probe_gbs
    result["cpu_baseline"] = None
    del wl
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, spec, main_run["T"], stacked)
    print(json.dumps(result), flush=True)


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
    gu = [n for n in fetch if args.traffic_kernel in n]
    if not gu:
        raise SystemExit(f"no kernel named like {args.traffic_kernel!r} in the counter CSV")
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
    config = meta.get("counters_run", "c4")
    out = {
        "config": config,
        "tokens": meta.get("tokens"),
        "kernel_source_hash": meta["kernel_source_hash"] if "kernel_source_hash" in meta else kernel_source_hash(),
        "bytes_per_launch": int(round(fb + wb)),
        "fetch_bytes_per_launch": int(round(fb)),
        "write_bytes_per_launch": int(round(wb)),
        "algorithmic_bytes_per_launch": meta.get("gateup_bytes_per_launch"),
        "calibration": {"copy_kernel": fname, "copy_bytes": COPY_BYTES, "fetch_kib": fcopy, "write_kib": wcopy,
                        "fetch_scale": f_scale, "write_scale": w_scale},
        "kernels": per_kernel,
    }
    with open(traffic_file(config), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, spec, T, stacked):
    """The oracle as it stands, on a bounded sample of the same workload: independent
    layer forwards of T tokens (seeded layer instances, each with its own input rows; for
    the stacked config each forward is one layer of the 36, teacher-forced), one per
    worker thread on every core the job may use, until about the time budget is spent.
    The stacked config's rate is the per-layer rate divided by the depth."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    import synth
    cores = min(16, len(os.sched_getaffinity(0)))

    def item(l):
        x = synth.make_x(spec, T=T, layer=l)
        router_only = synth.make_layer(spec, layer=l, experts=[])
        x64 = oracle.activations_f64(x, spec.x_dtype)
        ids, _ = oracle.topk_softmax(oracle.router_logits(x64, router_only.router_w, router_only.router_b),
                                     spec.top_k)
        return synth.make_layer(spec, layer=l, experts=np.unique(ids)), x

    def run(it):
        layer, x = it
        oracle.moe_forward(layer, x, spec.x_dtype)

    # one forward alone sizes the sample: rounds of one forward per core
    first = item(0)
    t0 = time.perf_counter()
    run(first)
    t_one = time.perf_counter() - t0
    rounds = max(1, int(round(args.cpu_seconds / max(t_one, 1e-3))))
    n_items = rounds * cores
    items = [item(l) for l in range(1, n_items + 1)]
    with ThreadPoolExecutor(cores) as ex:
        t0 = time.perf_counter()
        list(ex.map(run, items))
        wall = time.perf_counter() - t0
    log(args, f"cpu oracle: {n_items} layer forwards of {T} token(s) on {cores} threads in {wall:.1f} s "
              f"(one alone {t_one:.1f} s)")
    depth = spec.n_layers if stacked else 1
    tokens_per_s = T * n_items / wall / depth
    what = (f"{n_items} independent forwards of {T} token(s) through seeded instances of one layer, one per "
            f"worker thread, {wall:.1f} s wall" + (f"; per-layer rate divided by the {depth}-layer depth"
                                                   if stacked else "")
            + "; fp64 numpy oracle")
    return {"value": round(tokens_per_s, 5), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": what, "cpu_model": cpu_model(), "cores_available": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
