"""Benchmark of the routed-expert MoE layer on one MI355X.

One step = one pass of 48 MoE layers (each layer its own seeded weights,
activations and router logits, all resident in HBM), captured in a HIP graph
and replayed; every step runs the whole hot path (routing, grouping, expert
FFNs, shared expert, combine).

    python bench.py [--workload decode|mtp16|e512|e512x4|prefill|tiny] [--steps K] [--warmup W]

Prints one JSON line.  The default workload is the decode layer (one row per
window, 128 experts, top-8 + shared expert, 4-bit, hidden 2048, FFN 768).
`value` is the effective expert-weight bandwidth (distinct experts touched per
layer, plus the shared expert, each blob's bytes counted once) over the
whole pass; for the prefill workload it is tokens/s.  `roofline` rates the
dominant kernel against MI355X's HBM (8 TB/s) or bf16 MFMA (2.5 PFLOP/s)
peak from its own duration, timed with HIP events recorded on its stream
around each launch.  `cpu_baseline` is the CPU oracle timed on a bounded
sample of the same workload on this host.
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

WORKLOADS = {
    # name: (config, rows)
    "tiny": ("tiny", 4),
    "decode": ("decode", 1),
    "mtp16": ("mtp16", 16),
    "e512": ("e512", 1),
    "e512x4": ("e512", 4),
    "prefill": ("prefill", 2048),
}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode", choices=sorted(WORKLOADS))
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the layer's kernels run on one device); --gpus {args.gpus} "
              f"is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    from quantized_routed_expert_amd import moe, synth

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

    cname, T = WORKLOADS[args.workload]
    cfg = synth.CONFIGS[cname]
    L = args.layers
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    path = moe.PATH_DECODE if T <= moe.DECODE_MAX_ROWS else moe.PATH_PREFILL

    # ---- inputs: 48 independent layers, resident in HBM ----------------------
    t0 = time.time()
    layers = []
    host_keep = []  # a few layers kept on the host for the oracle sample
    eb = cfg.expert_bytes
    bytes_layer = []
    for l in range(L):
        li = synth.layer_inputs(cfg, layer=l, T=T)
        d = {
            "x": (torch.from_numpy(li.x.view(np.int16)).view(torch.bfloat16) if cfg.x_dtype == "bf16"
                  else torch.from_numpy(li.x)).to(dev),
            "logits": torch.from_numpy(li.logits).to(dev),
        }
        # weights converted once to the order the kernels read (outside the timed region)
        d["routed_t"], d["routed"] = moe.prepare_qweights(torch.from_numpy(li.routed).to(dev), cfg.bits,
                                                          cfg.n_experts, cfg.hidden, cfg.ffn)
        d["shared_t"], d["shared"] = (moe.prepare_qweights(torch.from_numpy(li.shared).to(dev), cfg.bits, 1,
                                                           cfg.hidden, cfg.shared_ffn)
                                      if li.shared is not None else (None, None))
        d["y"] = torch.empty((T, cfg.hidden), dtype=torch.float32, device=dev)
        nd = distinct_experts(li.logits, cfg.top_k)
        bytes_layer.append(nd * eb + cfg.shared_bytes)
        layers.append(d)
        if len(host_keep) < 48:
            host_keep.append(li)
        if l % 8 == 7 or l == L - 1:
            log(f"generated and uploaded {l + 1}/{L} layers ({time.time() - t0:.0f} s)")
    torch.cuda.synchronize()
    ws = moe.workspace(T, cfg.n_experts, cfg.top_k, cfg.hidden, cfg.ffn, cfg.shared_ffn, path)

    stream = torch.cuda.Stream()

    def one_pass(s):
        for d in layers:
            moe.layer_forward(d["x"], d["logits"], cfg.top_k, d["routed"], d["shared"], d["y"], ws, path=path,
                              stream=s)

    # ---- warmup (eager), then capture one pass --------------------------------
    with torch.cuda.stream(stream):
        for _ in range(max(args.warmup, 1)):
            one_pass(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            one_pass(stream)
    torch.cuda.synchronize()
    for _ in range(max(args.warmup, 1)):
        graph.replay()
    torch.cuda.synchronize()
    log("warmup done")

    # ---- timed region: K replays of the 48-layer pass ---------------------------
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
    log(f"pass {ms_step:.4f} ms, {us_layer:.2f} us/layer")

    # ---- dominant kernel's own duration.  Decode: the layer is one kernel
    # launch, so the timed region (events on the kernel's stream) over its K*L
    # launches is that kernel's average duration plus the graph's launch gap.
    # Prefill: events on the stream around each layer's launches.
    reps = 3
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(L * reps)]
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
    per_launch_us = np.array([a.elapsed_time(b) * 1000.0 for a, b in evs])
    kern_us = float(np.mean(per_launch_us))
    log(f"per-launch (event-bracketed) {kern_us:.2f} us")

    total_bytes = float(np.sum(bytes_layer))
    gbs = total_bytes / (ms_step * 1e-3) / 1e9
    toks = T * 1000.0 / ms_step  # tokens per second through a 48-layer MoE stack
    fl_gu, fl_dn = layer_flops(cfg, T)

    if path == moe.PATH_DECODE:
        metric_value, unit = gbs, "GB/s"
        kern_us = us_layer
        ach = (total_bytes / L) / (kern_us * 1e-6) / 1e9
        # windows of one to four rows (T * k <= 64) take the column-split
        # launch (integer nibble dot products), larger windows the matrix-core launch
        split = T <= 4 and T * cfg.top_k <= 64
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload),
                "kernel": "k_split_layer" if split else "k_decode_layer", "bytes_per_launch": round(total_bytes / L),
                "launch_us": round(kern_us, 3)}
        # split: signed 4-bit products (codes x 16-bit activation digits), int32
        # block sums, fp32 scale and accumulate; matrix-core: f16 MFMA, fp32 accumulate
        dtype = "i4" if split else "f16"
    else:
        metric_value, unit = toks, "tok/s"
        ach = (fl_gu + fl_dn) / (kern_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": measured_traffic(args.workload),
                "kernel": "layer (route, group, plan, gate/up GEMM, down GEMM, combine)",
                "flops_per_launch": fl_gu + fl_dn}
        dtype = "bf16"

    # ---- CPU baseline: the oracle on a bounded sample ------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.Oracle()
        t_start = time.time()
        n_layers = 0
        rows_done = 0
        cpu_bytes = 0.0
        if path == moe.PATH_DECODE:
            # the layers of the pass in order, cycling, until the time budget is spent
            while time.time() - t_start < args.cpu_seconds:
                li = host_keep[n_layers % len(host_keep)]
                orc.layer_forward(li.x, li.x_code, li.logits, cfg.top_k, cfg.bits, cfg.ffn, li.routed, li.shared,
                                  s_ffn=cfg.shared_ffn or None)
                cpu_bytes += bytes_layer[n_layers % len(host_keep)]
                n_layers += 1
            dt = time.time() - t_start
            cpu = {"value": round(cpu_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                   "sample": f"{n_layers} layer evaluations (the pass's {len(host_keep)} layers in order, "
                             f"cycling), all {T} row(s), single-threaded C oracle ({dt:.1f} s); "
                             f"{dt / n_layers * 1e6:.0f} us/layer"}
        else:
            li = host_keep[0]
            step = 16
            while time.time() - t_start < args.cpu_seconds and rows_done < T:
                rows = np.arange(rows_done, min(rows_done + step, T), dtype=np.int32)
                orc.layer_forward(li.x, li.x_code, li.logits, cfg.top_k, cfg.bits, cfg.ffn, li.routed, li.shared,
                                  s_ffn=cfg.shared_ffn or None, rows=rows)
                rows_done += rows.size
            dt = time.time() - t_start
            cpu = {"value": round(rows_done / dt / L, 4), "unit": "tok/s", "cores": 1, "kind": "oracle",
                   "sample": f"{rows_done} of the {T} chunk rows of layer 0 (routing of all rows), "
                             f"single-threaded C oracle ({dt:.1f} s), scaled to a {L}-layer pass"}
        log(f"cpu baseline {cpu['value']} {cpu['unit']}")

    out = {
        "metric": "MoE layer us + expert-weight GB/s at 1-16 decode rows; prefill tok/s",
        "value": round(metric_value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded; weights N(0,0.02) block-quantized, activations N(0,1), logits per recipe)",
        "config": {
            "workload": f"{args.workload}: H={cfg.hidden} E={cfg.n_experts} F={cfg.ffn} top-{cfg.top_k}"
                        f" + shared F={cfg.shared_ffn}, {cfg.bits}-bit block-32, T={T} rows, {L} layers",
            "rows": T, "layers": L, "path": "decode" if path == moe.PATH_DECODE else "prefill",
            "us_per_layer": round(us_layer, 3),
            "tokens_per_s": round(toks, 1),
            "expert_weight_GBps": round(gbs, 1),
            "mean_distinct_experts": round(float(np.mean([b - cfg.shared_bytes for b in bytes_layer]) / eb), 2),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
