"""Benchmark of the routed-expert MoE layer on one MI355X.

One step = one pass of 48 MoE layers (each layer its own seeded weights,
activations and router logits, all resident in HBM), captured in a HIP graph
and replayed; every step runs the whole hot path (routing, grouping, expert
FFNs, shared expert, combine).

    python bench.py [--workload all|decode|decode_router|tiny|mtp16|e512|e512x4|prefill|e512_nl4|prefill_nl4]
                    [--steps K] [--warmup W]

The default runs every workload (the five configurations; the
large-expert-count decode at 1 and 4 rows; the decode layer with its router
projection; the large-expert-count layer with a 3-bit gate/up and a
non-linear 4-bit down projection, at one row and as a prefill chunk) and
prints ONE JSON line.  Its
top-level fields are the decode workload's (one row per window, 128 experts,
top-8 + shared expert, 4-bit, hidden 2048, FFN 768); `workloads` lists every
workload with its us/layer, tokens/s, expert-weight GB/s, roofline fraction,
counter traffic and CPU baseline.  `value` is the effective expert-weight
bandwidth (distinct experts touched per layer, plus the shared expert, each
blob's bytes counted once) over the whole pass; for the prefill workload it
is tokens/s.  `roofline` rates the dominant kernel against MI355X's HBM
(8 TB/s) or bf16 MFMA (2.5 PFLOP/s) peak from its own duration, timed with
HIP events recorded on its stream.  `cpu_baseline` is the CPU oracle timed
on a bounded sample of the same workload on this host, on all cores (OpenMP
over rows) and on one.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "MoE layer us + expert-weight GB/s at 1-16 decode rows; prefill tok/s"

# the pairing of the thread's decode table: 3-bit gate/up, non-linear 4-bit
# down (the table is the test table 127 sign(t)|t|^1.6, t = (i - 7.5)/7.5)
_NL4_DOWN = {"down_bits": 20, "codebook": None}  # codebook filled in by workload_config

# name: (config, rows[, format changes]); the order of the default run (the headline first)
WORKLOADS = {
    "decode": ("decode", 1),
    # the decode layer with its router projection (bf16 [E][H]) in the same
    # captured 48-layer graph: the logits come from x instead of the recipe
    "decode_router": ("decode", 1),
    "tiny": ("tiny", 4),
    "mtp16": ("mtp16", 16),
    "e512": ("e512", 1),
    "e512x4": ("e512", 4),
    "prefill": ("prefill", 2048),
    "e512_nl4": ("e512", 1, _NL4_DOWN),
    "prefill_nl4": ("prefill", 2048, _NL4_DOWN),
}
ROUTER_WORKLOADS = {"decode_router"}


def workload_config(name):
    """(config, rows) of a workload, its format changes applied."""
    import dataclasses
    from quantized_routed_expert_amd import synth
    spec = WORKLOADS[name]
    cfg = synth.CONFIGS[spec[0]]
    if len(spec) > 2:
        ch = dict(spec[2])
        if ch.get("codebook", ()) is None:
            ch["codebook"] = synth.nl4_test_codebook()
        cfg = dataclasses.replace(cfg, name=name, **ch)
    return cfg, spec[1]


def format_desc(cfg) -> str:
    def one(b):
        return "non-linear 4-bit" if b == 20 else f"{b}-bit"
    if cfg.dbits == cfg.bits:
        return f"{one(cfg.bits)} block-32"
    return f"gate/up {one(cfg.bits)}, down {one(cfg.dbits)} block-32"


def weight_key(cfg):
    return (cfg.wcid, cfg.bits, cfg.dbits, tuple(cfg.codebook), cfg.hidden, cfg.ffn, cfg.n_experts, cfg.shared_ffn)


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def distinct_experts(logits: np.ndarray, k: int) -> int:
    """Experts a window touches: the union of each row's top-k (ids compared as
    the router does: largest fp32 logit, ties to the lower id)."""
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :k]
    return int(np.unique(order).size)


def source_digest() -> str:
    """sha256 over the HIP sources and the ABI header: identifies the kernel
    build that a stored counter summary belongs to."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_routed_expert_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    with open(os.path.join(ROOT, "include", "moe.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter
    reads for a plain copy of known size), or None when there is no summary for
    this workload or the kernel sources have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic.{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("source_digest") != source_digest():
        return None
    try:
        return round(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def layer_flops(cfg, T: int) -> tuple[float, float]:
    """(gate/up FLOPs, down FLOPs) of one layer: 2*H*F per matrix per routed
    row, for T*k routed rows plus T shared rows."""
    routed = T * cfg.top_k * cfg.hidden * cfg.ffn * 2.0
    shared = T * cfg.hidden * cfg.shared_ffn * 2.0
    return 2 * (routed + shared), routed + shared


def host_info() -> dict:
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"nproc": usable, "cpu_count": os.cpu_count(), "cpu_model": model,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


class WeightCache:
    """Prepared weight sets on the device, shared by the workloads that read
    the same layer weights (e512, e512x4 and prefill), freed when no later
    workload needs them."""

    def __init__(self, dev, layers: int):
        self.dev = dev
        self.layers = layers
        self.sets = {}

    def get(self, cfg):
        import torch
        from quantized_routed_expert_amd import moe, synth
        key = weight_key(cfg)
        if key in self.sets:
            return self.sets[key]
        t0 = time.time()
        out = []
        for l in range(self.layers):
            raw = synth.routed_weights_torch(cfg, l, self.dev)
            cb = cfg.codebook or None
            routed_t, routed = moe.prepare_qweights(raw, cfg.bits, cfg.n_experts, cfg.hidden, cfg.ffn,
                                                    down_bits=cfg.down_bits, codebook=cb)
            sh = synth.shared_weights(cfg, l)
            shared_raw = torch.from_numpy(sh).to(self.dev) if sh is not None else None
            shared_t, shared = (moe.prepare_qweights(shared_raw, cfg.bits, 1, cfg.hidden, cfg.shared_ffn,
                                                     down_bits=cfg.down_bits, codebook=cb)
                                if sh is not None else (None, None))
            # the pages' block order of a few layers stays on the host for the oracle
            host = (raw.cpu().numpy(), sh) if l < 4 else None
            del raw, shared_raw
            out.append({"routed_t": routed_t, "routed": routed, "shared_t": shared_t, "shared": shared,
                        "host": host})
        torch.cuda.synchronize()
        log(f"weights of {cfg.name}-shaped layers: {self.layers} layers generated and prepared on the device "
            f"({time.time() - t0:.1f} s)")
        self.sets[key] = out
        return out

    def drop_unless(self, cfgs_left):
        import torch
        keep = {weight_key(c) for c in cfgs_left}
        for key in list(self.sets):
            if key not in keep:
                del self.sets[key]
        torch.cuda.empty_cache()


def cpu_baseline(orc, cfg, T, wsets, xs, logits, bytes_layer, seconds, path_decode, L, routers=None):
    """The oracle on a bounded sample of the workload, on all cores (OpenMP
    over rows) and on one; returns the cpu_baseline object.  With routers
    (bf16 router matrices), each layer evaluation starts from the router
    projection."""
    nthreads = orc.set_threads(0)
    res = {}
    for leg, nt in (("all_cores", nthreads), ("one_core", 1)):
        orc.set_threads(nt)
        t_start = time.time()
        if path_decode:
            n_layers, cpu_bytes = 0, 0.0
            while time.time() - t_start < seconds or n_layers == 0:
                l = n_layers % min(4, L)
                routed, shared = wsets[l]["host"]
                lg = logits[l]
                if routers is not None:
                    lg = orc.router_logits(xs[l], 0 if cfg.x_dtype == "f32" else 1, routers[l]).astype(np.float32)
                orc.layer_forward(xs[l], 0 if cfg.x_dtype == "f32" else 1, lg, cfg.top_k, cfg.fmt,
                                  cfg.ffn, routed, shared, s_ffn=cfg.shared_ffn or None,
                                  codebook=cfg.codebook or None)
                cpu_bytes += bytes_layer[l]
                n_layers += 1
            dt = time.time() - t_start
            res[leg] = {"value": round(cpu_bytes / dt / 1e9, 4), "unit": "GB/s", "threads": nt,
                        "us_per_layer": round(dt / n_layers * 1e6, 1),
                        "sample": f"{n_layers} layer evaluations of {T} row(s) (layers 0-3 of the pass, "
                                  f"cycling), {dt:.1f} s"}
        else:
            routed, shared = wsets[0]["host"]
            step = 16 if nt == 1 else 256
            rows_done = 0
            while (time.time() - t_start < seconds or rows_done == 0) and rows_done < T:
                rows = np.arange(rows_done, min(rows_done + step, T), dtype=np.int32)
                orc.layer_forward(xs[0], 0 if cfg.x_dtype == "f32" else 1, logits[0], cfg.top_k, cfg.fmt,
                                  cfg.ffn, routed, shared,
                                  s_ffn=cfg.shared_ffn or None, rows=rows, codebook=cfg.codebook or None)
                rows_done += rows.size
            dt = time.time() - t_start
            res[leg] = {"value": round(rows_done / dt / L, 4), "unit": "tok/s", "threads": nt,
                        "sample": f"{rows_done} of the {T} chunk rows of layer 0 (routing of all rows), "
                                  f"{dt:.1f} s, scaled to a {L}-layer pass"}
    orc.set_threads(nthreads)
    main = res["all_cores"]
    return {"value": main["value"], "unit": main["unit"], "cores": nthreads, "kind": "oracle",
            "sample": main["sample"] + "; C oracle, OpenMP over rows", "one_core": res["one_core"],
            **host_info()}


def run_workload(name, args, wcache, orc):
    import torch
    from quantized_routed_expert_amd import moe, synth

    cfg, T = workload_config(name)
    L = args.layers
    dev = wcache.dev
    path = moe.PATH_DECODE if T <= moe.DECODE_MAX_ROWS else moe.PATH_PREFILL

    # ---- inputs: L independent layers, resident in HBM ------------------------
    wsets = wcache.get(cfg)
    router = name in ROUTER_WORKLOADS
    xs, lgs, layers, bytes_layer, routers = [], [], [], [], []
    eb = cfg.expert_bytes
    for l in range(L):
        x = synth.activations(cfg, l, T)
        xs.append(x)
        d = dict(wsets[l])
        d["x"] = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if cfg.x_dtype == "bf16"
                  else torch.from_numpy(x)).to(dev)
        if router:
            wr = synth.router_weights(cfg, l)
            routers.append(wr)
            d["w_router"] = torch.from_numpy(wr.view(np.int16)).view(torch.bfloat16).to(dev)
            d["logits"] = moe.router_logits(d["x"], d["w_router"])
            lg = d["logits"].cpu().numpy()
        else:
            lg = synth.logits(cfg, l, T)
            d["logits"] = torch.from_numpy(lg).to(dev)
        lgs.append(lg)
        d["y"] = torch.empty((T, cfg.hidden), dtype=torch.float32, device=dev)
        bytes_layer.append(distinct_experts(lg, cfg.top_k) * eb + cfg.shared_bytes)
        layers.append(d)
    torch.cuda.synchronize()
    ws = moe.workspace(T, cfg.n_experts, cfg.top_k, cfg.hidden, cfg.ffn, cfg.shared_ffn, path)
    stream = torch.cuda.Stream()

    def one_pass(s):
        for d in layers:
            if router:
                moe.router_logits(d["x"], d["w_router"], logits=d["logits"], stream=s)
            moe.layer_forward(d["x"], d["logits"], cfg.top_k, d["routed"], d["shared"], d["y"], ws, path=path,
                              stream=s)

    # ---- warmup (eager), then capture one pass --------------------------------
    with torch.cuda.stream(stream):
        for _ in range(max(args.warmup, 1)):
            one_pass(stream)
    torch.cuda.synchronize()
    assert moe.workspace_error(ws) == 0, "device error word set during warmup"
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            one_pass(stream)
    torch.cuda.synchronize()
    for _ in range(max(args.warmup, 1)):
        graph.replay()
    torch.cuda.synchronize()

    # ---- timed region: K replays of the L-layer pass ----------------------------
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    us_layer = ms_step * 1000.0 / L
    err = moe.workspace_error(ws)
    assert err == 0, f"device error word {err} after the timed region"
    log(f"{name}: pass {ms_step:.4f} ms, {us_layer:.2f} us/layer")

    total_bytes = float(np.sum(bytes_layer))
    gbs = total_bytes / (ms_step * 1e-3) / 1e9
    toks = T * 1000.0 / ms_step  # tokens per second through an L-layer MoE stack
    fl_gu, fl_dn = layer_flops(cfg, T)
    desc = (f"{name}: H={cfg.hidden} E={cfg.n_experts} F={cfg.ffn} top-{cfg.top_k} + shared F={cfg.shared_ffn}, "
            f"{format_desc(cfg)}, T={T} rows, {L} layers"
            + (f", bf16 router projection [{cfg.n_experts}][{cfg.hidden}] per layer in the graph" if router else ""))

    if path == moe.PATH_DECODE:
        metric_value, unit = gbs, "GB/s"
        # the layer is one kernel launch: the timed region (events on the
        # kernel's stream) over its K*L launches is that kernel's average
        # duration plus the graph's launch gap
        kern_us = us_layer
        ach = (total_bytes / L) / (kern_us * 1e-6) / 1e9
        # windows of one to four rows (T * k <= 64) take the column-split
        # launch (integer nibble dot products), larger windows the matrix-core launch
        split = T <= 4 and T * cfg.top_k <= 64 and cfg.bits in (3, 4) and cfg.dbits in (3, 4)
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(name),
                "kernel": "k_split_layer" if split else "k_decode_layer", "bytes_per_launch": round(total_bytes / L),
                "launch_us": round(kern_us, 3)}
        if router:
            # the pass holds two launches per layer: the rate covers both
            roof["kernel"] += " + k_router_logits"
            roof["router_bytes_per_layer"] = cfg.n_experts * cfg.hidden * 2
        # split: signed 4-bit products (codes x 15-bit integer activations cut
        # into signed radix-16 digits), int32 block sums, fp32 scale and
        # accumulate; matrix-core: f16 MFMA on exact codes and hi+lo activations
        dtype = "i4" if split else "f16"
    else:
        metric_value, unit = toks, "tok/s"
        # events on the stream around each layer's launches (route, group,
        # plan, both GEMMs, combine)
        reps = 2
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(L * reps)]
        with torch.cuda.stream(stream):
            i = 0
            for _ in range(reps):
                for d in layers:
                    evs[i][0].record(stream)
                    moe.layer_forward(d["x"], d["logits"], cfg.top_k, d["routed"], d["shared"], d["y"], ws,
                                      path=path, stream=stream)
                    evs[i][1].record(stream)
                    i += 1
        torch.cuda.synchronize()
        kern_us = float(np.mean([a.elapsed_time(b) * 1000.0 for a, b in evs]))
        ach = (fl_gu + fl_dn) / (kern_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": measured_traffic(name),
                "kernel": "layer (route, group, plan, gate/up GEMM, down GEMM, combine)",
                "flops_per_launch": fl_gu + fl_dn, "launch_us": round(kern_us, 3),
                "hbm_frac_of_weights": round((total_bytes / L) / (kern_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        dtype = "bf16"

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(orc, cfg, T, wsets, xs, lgs, bytes_layer, args.cpu_seconds,
                           path == moe.PATH_DECODE, L, routers if router else None)
        log(f"{name}: cpu baseline {cpu['value']} {cpu['unit']} on {cpu['cores']} threads, "
            f"{cpu['one_core']['value']} on one")

    return {
        "workload": name,
        "metric_value": round(metric_value, 3), "unit": unit, "ms_per_step": round(ms_step, 5), "dtype": dtype,
        "config": {"workload": desc, "rows": T, "layers": L,
                   "path": "decode" if path == moe.PATH_DECODE else "prefill",
                   "us_per_layer": round(us_layer, 3), "tokens_per_s": round(toks, 1),
                   "expert_weight_GBps": round(gbs, 1),
                   "mean_distinct_experts": round(float(np.mean([b - cfg.shared_bytes for b in bytes_layer]) / eb),
                                                  2),
                   "useful_TFLOPs": round((fl_gu + fl_dn) / (us_layer * 1e-6) / 1e12, 3)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all", choices=["all"] + list(WORKLOADS))
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=6.0, help="budget of each oracle leg per workload")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the layer's kernels run on one device); --gpus {args.gpus} "
              f"is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n,
                          "copies": 5}), flush=True)
        return

    from quantized_routed_expert_amd import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    names = list(WORKLOADS) if args.workload == "all" else [args.workload]
    orc = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.Oracle()
    wcache = WeightCache(dev, args.layers)
    results = []
    for i, name in enumerate(names):
        results.append(run_workload(name, args, wcache, orc))
        wcache.drop_unless([workload_config(n)[0] for n in names[i + 1:]])

    head = results[0]
    out = {
        "metric": METRIC,
        "value": head["metric_value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded; weights N(0,0.02) block-quantized, activations N(0,1), logits per recipe)",
        "config": head["config"],
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        "workloads": [{k: v for k, v in r.items()} for r in results],
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
