"""Benchmark of the causal block-scaled MXFP8 attention training call on one
MI355X: quantize + forward + backward over packed documents, inputs resident
in HBM, one JSON line on stdout.

A step is one whole call (flamia_quantize, flamia_attn_fwd, flamia_attn_bwd;
the timed steps are replays of the step captured once in a HIP graph, with the
eager timing beside them)
over the 2 x 4096-token, 16-head, head-dim-128 workload with 1% outlier
channels and the Hadamard rotation on.  Throughput counts the algorithmic
causal FLOPs, 14 * d per (query, key) pair with key <= query inside a
document (forward 2 products, backward 5); quantization adds no FLOPs but
its time is inside the step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]
                       [--kv-heads Hk] [--deterministic] [--exact] [--non-causal]
                       [--causal-dq-scale] [--no-cpu-baseline]
                       [--copy-calibration]
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

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 matrix-core peak (published)
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak (published)
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E bandwidth (published)
CPU_SAMPLE_HEADS = 8          # oracle sample: document 0, this many heads (about 10-20 s)
METRIC = "fwd+bwd attention call ms & TFLOP/s incl. quantization; % of MFMA FP8 peak"
KERNEL_SOURCES = {
    "attn_bwd8_kernel": "precision_causal_attention_hadamard_amd/csrc/attn_bwd.hip",   # MXFP8 path
    "attn_bwd_kernel": "precision_causal_attention_hadamard_amd/csrc/attn_bwd.hip",    # mixed path
    "attn_fwd_kernel": "precision_causal_attention_hadamard_amd/csrc/attn_fwd.hip",
    "quant_qkv_kernel": "precision_causal_attention_hadamard_amd/csrc/quant.hip",
}


def source_hash(path: str) -> str:
    h = hashlib.sha256()
    for p in (path, "precision_causal_attention_hadamard_amd/csrc/flamia_device.hpp"):
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


def weighted_peak(parts):
    """Peak of a kernel whose products run in several dtypes: total FLOPs over
    the time each part would take at its own dtype's peak."""
    total = sum(f for f, _ in parts)
    return total / sum(f / p for f, p in parts)


def product_mix(d: int, pairs: int, mixed: bool):
    """(FLOPs, peak) per product dtype for the forward and the backward.
    Forward: S and P.V; backward: S again, dP, dV, dK, dQ (2 d per pair each).
    dV runs on bf16 MFMA (1/l rides in G); on the mixed path the S products
    are bf16 (expanded NVFP4)."""
    u = 2 * d * pairs
    s_peak = BF16_PEAK_TFLOPS if mixed else FP8_PEAK_TFLOPS
    fwd = [(u, s_peak), (u, FP8_PEAK_TFLOPS)]
    bwd = [(u, s_peak), (u, BF16_PEAK_TFLOPS), (3 * u, FP8_PEAK_TFLOPS)]
    return fwd, bwd


def _pmc_rows(run_dir: str, counter: str):
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    rows = []
    for fn in files:
        with open(fn) as f:
            rows += [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
    return rows


def write_traffic(fetch_dir: str, write_dir: str, cfg: int, command: str, kernel: str):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE, both with --copy-calibration) into the traffic record of the
    backward kernel.  Each counter is scaled by what it reads for the 1 GiB
    device copy in the same run (known bytes: 1 GiB read, 1 GiB written)."""
    rec = {"kernel": kernel, "workload": f"config{cfg}", "command": command,
           "source_sha": source_hash(KERNEL_SOURCES[kernel])}
    total = 0.0
    for counter, run_dir in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _pmc_rows(run_dir, counter)
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        if not copies:
            raise SystemExit(f"{counter}: no device copy in {run_dir} (run with --copy-calibration)")
        copy_kib = max(copies)
        factor = (1 << 30) / 1024.0 / copy_kib
        vals = [float(r["Counter_Value"]) for r in rows if f"flamia::{kernel}<" in r["Kernel_Name"]]
        if not vals:
            raise SystemExit(f"{counter}: no {kernel} dispatch in {run_dir}")
        kib = sum(vals) / len(vals)
        rec[counter] = {"kib_per_dispatch_raw": kib, "dispatches": len(vals),
                        "copy_1GiB_reads_kib": copy_kib, "scale": factor,
                        "bytes_per_launch": kib * 1024.0 * factor}
        total += kib * 1024.0 * factor
    rec["hbm_bytes_per_launch"] = total
    path = os.path.join(ROOT, "profiles", f"{kernel}_config{cfg}_traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def toolchain(torch):
    """Versions the numbers depend on (the pages warn that results drift
    with toolchain versions)."""
    import subprocess
    info = {"torch": torch.__version__, "hip_runtime": getattr(torch.version, "hip", None)}
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    try:
        r = subprocess.run(["/opt/rocm/bin/hipcc", "--version"], capture_output=True, text=True, timeout=30)
        info["hipcc"] = next((l.strip() for l in r.stdout.splitlines() if "HIP version" in l), None)
    except (OSError, subprocess.SubprocessError):
        info["hipcc"] = None
    info["device"] = torch.cuda.get_device_name(0)
    info["arch"] = getattr(torch.cuda.get_device_properties(0), "gcnArchName", None)
    return info


def graph_replay(call, torch, steps: int, warmup: int, flops: int):
    """The same step captured once in a HIP graph and replayed (the pages time
    the call this way): K timed replays after W warm-ups, bracketed by
    synchronisations; reported beside the eager timing."""
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call.step()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        return {"ms_per_step": ms, "TFLOP/s": flops / (ms * 1e-3) / 1e12, "replays": steps}
    except RuntimeError as e:      # reported, never fatal to the eager measurement
        return {"error": str(e)[:200]}


def worklist_build(flamia, torch, ndocs: int = 131072):
    """The GPU work-list build alone (flamia_plan_build) on the pages' stress
    case: ndocs single-token documents.  HIP events on the launch stream,
    median of 20 builds after 3 warm-ups."""
    dev = torch.device("cuda:0")
    z = torch.zeros(ndocs, 1, 64, dtype=torch.bfloat16, device=dev)
    call = flamia.TrainingCall(z, z, z, z, list(range(ndocs + 1)))
    for _ in range(3):
        flamia.plan_build(call.desc, call.qt)
    ms = []
    for _ in range(20):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flamia.plan_build(call.desc, call.qt)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    ms.sort()
    fwd, bwd = call.plan_lists()
    return {"docs": ndocs, "tokens": ndocs, "ms": ms[len(ms) // 2], "fwd_items": len(fwd), "bwd_items": len(bwd)}


def cpu_baseline(wl, cfg: int, causal: bool = True):
    """The oracle, as it stands, on document 0 and the first few heads of the
    workload, timed on the host cores."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention as A

    s, e = wl.cu_seqlens[0], wl.cu_seqlens[1]
    g = wl.heads // wl.kv_heads                       # query heads per key/value head
    nh = max(g, min(CPU_SAMPLE_HEADS, wl.heads) // g * g)
    arrs = [t[s:e, 0:(nh if t.shape[1] == wl.heads else nh // g)].float().numpy().astype(np.float64)
            for t in (wl.q, wl.k, wl.v, wl.do)]
    L = e - s
    t0 = time.perf_counter()
    A.training_call(*arrs, [0, L], A.Numerics(hadamard=wl.hadamard, path="mixed" if wl.path else "mxfp8",
                                              causal=causal))
    dt = time.perf_counter() - t0
    flops = 14 * wl.head_dim * nh * (L * (L + 1) // 2 if causal else L * L)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"document 0 ({L} tokens), heads 0-{nh - 1} of the {wl.name} workload: "
                      f"quantize+fwd+bwd, {dt:.2f} s; fp64 numpy, BLAS threads={threads}, "
                      "elementwise steps single-threaded",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="grouped-query variant of the workload: K and V with this many heads (0: one per query head)")
    ap.add_argument("--exact", action="store_true",
                    help="the exact option: per-token scales, all-tile V fold, per-row/per-key dS exponents")
    ap.add_argument("--non-causal", action="store_true",
                    help="the call without the causal mask (every key of a document visible); "
                         "FLOPs then count every (query, key) pair of a document")
    ap.add_argument("--causal-dq-scale", action="store_true",
                    help="the optional causal dQ accumulator scale (prescale from causally visible key blocks only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--deterministic", action="store_true",
                    help="ordered dQ reduction (per-step partials, fixed-order fp16 sum) instead of atomics")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (known bytes) for counter calibration")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: write the backward kernel's traffic record from two rocprofv3 --pmc runs")
    ap.add_argument("--pmc-command", default="",
                    help="with --write-traffic: the rocprofv3 command that made the runs")
    ap.add_argument("--traffic-kernel", default="attn_bwd8_kernel",
                    help="with --write-traffic: the kernel whose dispatches are summed")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic, args.config, args.pmc_command, args.traffic_kernel)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the call would shard by heads/documents with no exchange, which is not built.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from precision_causal_attention_hadamard_amd import flamia, workloads

    flamia.load()
    wl = workloads.config(args.config, kv_heads=args.kv_heads)
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.do))
    call = flamia.TrainingCall(q, k, v, do, wl.cu_seqlens, hadamard=wl.hadamard,
                               causal_dq_scale=wl.causal_dq_scale or args.causal_dq_scale, path=wl.path,
                               deterministic=args.deterministic, exact=args.exact,
                               causal=not args.non_causal)
    T, H, d = call.shape
    Hk = call.kv_heads
    grouped = Hk != H
    if args.non_causal:
        pairs = H * sum(L * L for L in wl.doc_lens)
        flops = 14 * d * pairs
    else:
        pairs = wl.causal_pairs()
        flops = wl.flops()

    def step(ev=None):
        if ev is not None: ev[0].record()
        call.quantize()
        if ev is not None: ev[1].record()
        call.forward()
        if ev is not None: ev[2].record()
        flamia.attn_bwd_prep(call.desc, call.qt, call.o, call.row_max, call.row_sum, call.do, call.bws)
        if ev is not None: ev[3].record()
        flamia.attn_bwd_main(call.desc, call.qt, call.dk, call.dv, call.bws)
        if ev is not None: ev[4].record()
        flamia.attn_bwd_finish(call.desc, call.qt, call.dq, call.dk, call.bws)
        if ev is not None: ev[5].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    names = ["quantize", "attn_fwd", "bwd_prep", "attn_bwd", "bwd_finish"]
    stage_ms = {n: sum(ev[i].elapsed_time(ev[i + 1]) for ev in events) / args.steps
                for i, n in enumerate(names)}
    event_ms = sum(stage_ms.values())
    eager_ms = ms_per_step
    # the headline: the same step captured once in a HIP graph and replayed K
    # times (how the pages time the call); eager timing if capture fails
    graph = graph_replay(call, torch, args.steps, args.warmup, flops)
    timing = "eager"
    if "ms_per_step" in graph:
        ms_per_step, timing = graph["ms_per_step"], "hip_graph_replay"
    value = flops / (ms_per_step * 1e-3) / 1e12

    # roofline of the dominant kernel
    E, Ek = T * H * d, T * Hk * d
    # quantizer bytes: bf16 Q, K, V read; Q, K, V, per-key V codes written;
    # one exponent byte per token and head of Q and four planes of the K side
    qbytes = 3 * E + 7 * Ek + T * H + 4 * T * Hk
    fwd_mix, bwd_mix = product_mix(d, pairs, bool(wl.path))
    kernels = {
        "attn_bwd": ("attn_bwd_kernel" if wl.path else "attn_bwd8_kernel", "mfma", 10 * d * pairs,
                     weighted_peak(bwd_mix)),
        "attn_fwd": ("attn_fwd_kernel", "mfma", 4 * d * pairs, weighted_peak(fwd_mix)),
        "quantize": ("quant_qkv_kernel", "hbm", qbytes, HBM_PEAK_GBS),
    }
    dom = max(kernels, key=lambda n: stage_ms[n])
    kname, bound, work, peak = kernels[dom]
    t_dom = stage_ms[dom] * 1e-3
    if bound == "mfma":
        achieved, unit = work / t_dom / 1e12, "TFLOP/s"
    else:
        achieved, unit = work / t_dom / 1e9, "GB/s"
    traffic = (measured_traffic(kname, f"config{args.config}")
               if kname.startswith("attn_bwd") and not grouped and not args.exact and not args.non_causal
               else None)
    roofline = {"bound": bound, "kernel": kname, "achieved": achieved, "peak": peak, "unit": unit,
                "frac": achieved / peak, "traffic": traffic,
                "peak_note": "dtype-weighted: FP8 products at 5000, bf16 products at 2500 TFLOP/s"
                             if bound == "mfma" else "HBM3E",
                "frac_of_fp8_peak": achieved / FP8_PEAK_TFLOPS if bound == "mfma" else None,
                "algorithmic_work_per_launch": work, "avg_launch_ms": stage_ms[dom]}
    quant = {"GB/s": qbytes / (stage_ms["quantize"] * 1e-3) / 1e9,
             "frac_hbm_peak": qbytes / (stage_ms["quantize"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
             "algorithmic_bytes": qbytes, "launches": 3 if wl.path else 2}

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": wl.name, "tokens": T, "heads": H, "kv_heads": Hk, "head_dim": d,
                   "doc_lens": wl.doc_lens if len(wl.doc_lens) <= 8 else f"{len(wl.doc_lens)} documents",
                   "hadamard": bool(wl.hadamard), "path": "mixed" if wl.path else "mxfp8",
                   "deterministic": bool(args.deterministic), "exact": bool(args.exact),
                   "causal": not args.non_causal, "causal_dq_scale": bool(wl.causal_dq_scale or args.causal_dq_scale),
                   "causal_pairs": pairs, "flops_per_step": flops},
        "pct_fp8_peak": 100.0 * value / FP8_PEAK_TFLOPS,
        "stage_ms": stage_ms, "event_ms_per_step": event_ms,
        # the attention kernels alone: forward, and backward without the dO
        # quantization / D preparation (quantization excluded on both sides)
        "kernel_only_ms": {"fwd": stage_ms["attn_fwd"], "bwd": stage_ms["attn_bwd"] + stage_ms["bwd_finish"]},
        "quantizer": quant,
        "roofline": roofline,
    }
    out["toolchain"] = toolchain(torch)
    out["timing"] = timing
    out["eager_ms_per_step"] = eager_ms
    out["graph"] = graph
    out["worklist"] = worklist_build(flamia, torch)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.config, causal=not args.non_causal)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
