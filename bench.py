"""Benchmark of the causal block-scaled MXFP8 attention training call on one
MI355X: quantize + forward + backward over packed documents, inputs resident
in HBM, one JSON line on stdout.

A step is one whole call (flamia_quantize, flamia_attn_fwd, flamia_attn_bwd),
captured once in a HIP graph and replayed: W warm-up replays, then 3 rounds
of exactly K timed replays, each bracketed by synchronisations; the median
round is the headline (the eager timing and per-stage HIP events are beside
it).  The default workload is the packed-document call: 4 rows x 16384
tokens of lognormal-length documents, 16 heads, head dim 128; the
long-context workload (2 x 12288 + short documents, 32768 tokens) is timed
after it with and without the causal dQ scale and reported under "extra".
Throughput counts the algorithmic causal FLOPs, 14 * d per (query, key) pair
with key <= query inside a document (forward 2 products, backward 5);
quantization adds no FLOPs but its time is inside the step.  The CPU
baseline (the oracle on a bounded sample, on the host's cores) runs first,
before the GPU is touched.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]
                       [--kv-heads Hk] [--deterministic] [--exact] [--non-causal]
                       [--causal-dq-scale] [--no-cpu-baseline] [--no-extra]
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
CPU_SAMPLE_MAX_LEN = 2048     # oracle sample: documents of at most this many tokens, all heads
CPU_WORKERS = 16              # worker processes of the CPU baseline: the GPU's share of a box
METRIC = "fwd+bwd attention call ms & TFLOP/s incl. quantization; % of MFMA FP8 peak"
KERNEL_SOURCES = {
    "attn_bwd8_kernel": "precision_causal_attention_hadamard_amd/csrc/attn_bwd.hip",   # MXFP8 path
    "attn_bwd_kernel": "precision_causal_attention_hadamard_amd/csrc/attn_bwd.hip",    # mixed path
    "attn_fwd_kernel": "precision_causal_attention_hadamard_amd/csrc/attn_fwd.hip",
    "quant_qkv_kernel": "precision_causal_attention_hadamard_amd/csrc/quant.hip",
    "finalize_dq_det_kernel": "precision_causal_attention_hadamard_amd/csrc/finalize.hip",   # deterministic dQ
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


def is_diag_instantiation(name: str) -> bool:
    """The backward's diagnostic instantiation (DIAG, the sixth template
    argument of attn_bwd8_kernel) writes extra counts; the bench launches it
    once for the dS zero fraction, and it is no launch of the timed kernel."""
    if "attn_bwd8_kernel<" not in name:
        return False
    args = name.split("attn_bwd8_kernel<", 1)[1].split(">", 1)[0].split(",")
    return len(args) > 5 and args[5].strip() == "true"


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
        vals = [float(r["Counter_Value"]) for r in rows
                if f"flamia::{kernel}<" in r["Kernel_Name"] and not is_diag_instantiation(r["Kernel_Name"])]
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
    with toolchain versions).  Read from files: nothing is started as a child
    process once the GPU is in use."""
    import re
    info = {"torch": torch.__version__, "hip_runtime": getattr(torch.version, "hip", None)}
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    try:
        with open("/opt/rocm/include/hip/hip_version.h") as f:
            h = f.read()
        v = [re.search(rf"#define HIP_VERSION_{k}\s+(\S+)", h) for k in ("MAJOR", "MINOR", "PATCH")]
        info["hip_headers"] = ".".join(m.group(1) for m in v) if all(v) else None
    except OSError:
        info["hip_headers"] = None
    info["device"] = torch.cuda.get_device_name(0)
    info["arch"] = getattr(torch.cuda.get_device_properties(0), "gcnArchName", None)
    return info


def timed_rounds(run, torch, steps: int, rounds: int = 3):
    """``rounds`` rounds of exactly ``steps`` calls of ``run``, each bracketed
    by synchronisations; ms per step of every round."""
    out = []
    for _ in range(rounds):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            run()
        torch.cuda.synchronize()
        out.append((time.perf_counter() - t0) * 1e3 / steps)
    return out


def graph_replay(call, torch, steps: int, warmup: int, flops: int):
    """The same step captured once in a HIP graph and replayed (the pages time
    the call this way): W warm-up replays, then 3 rounds of K timed replays,
    median round reported; beside the eager timing."""
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call.step()
        for _ in range(warmup):
            g.replay()
        rounds = timed_rounds(g.replay, torch, steps)
        ms = sorted(rounds)[len(rounds) // 2]
        return {"ms_per_step": ms, "TFLOP/s": flops / (ms * 1e-3) / 1e12, "replays_per_round": steps,
                "round_ms": rounds}
    except RuntimeError as e:      # reported, never fatal to the eager measurement
        return {"error": str(e)[:200]}


def p4_forward_timing(flamia, torch, wl, reps: int = 20):
    """The forward with the 4-bit probability operand (flamia_attn_fwd_p4)
    beside the plain forward on the same quantized operands: HIP events on the
    launch stream around each launch, median of ``reps`` after 3 warm-ups."""
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.do))
    call = flamia.TrainingCall(q, k, v, do, wl.cu_seqlens, hadamard=wl.hadamard)
    call.quantize()

    def med(fn):
        for _ in range(3):
            fn()
        ms = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return sorted(ms)[len(ms) // 2]

    f8 = med(call.forward)
    f4 = med(lambda: flamia.attn_fwd_p4(call.desc, call.qt, call.o, call.row_max, call.row_sum, call.fws))
    del call
    return {"workload": wl.name, "fwd_ms": f8, "fwd_p4_ms": f4, "p4_over_fp8": f4 / f8,
            "note": "4-bit probability operand (log-domain NVFP4, groups of 16 keys) carried into the FP8 P^V product"}


def worklist_build(flamia, torch, ndocs: int = 131072):
    """The GPU work-list build alone (flamia_plan_build) on the pages' stress
    case: ndocs single-token documents.  HIP events on the launch stream,
    median of 20 builds after 3 warm-ups."""
    dev = torch.device("cuda:0")
    z = torch.zeros(ndocs, 1, 64, dtype=torch.bfloat16, device=dev)
    call = flamia.TrainingCall(z, z, z, z, list(range(ndocs + 1)))
    ms = plan_build_ms(flamia, torch, call)
    fwd, bwd = call.plan_lists()
    return {"docs": ndocs, "tokens": ndocs, "ms": ms, "fwd_items": len(fwd), "bwd_items": len(bwd)}


def plan_build_ms(flamia, torch, call, reps: int = 20):
    """Median of ``reps`` work-list builds of a call (HIP events on the launch
    stream, after 3 warm-ups)."""
    for _ in range(3):
        flamia.plan_build(call.desc, call.qt)
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flamia.plan_build(call.desc, call.qt)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    ms.sort()
    return ms[len(ms) // 2]


def _oracle_unit(args):
    """One (document, heads) unit of the CPU baseline, in a worker process
    with single-threaded BLAS."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import attention as A
    arrs, L, hadamard, path, causal = args
    with threadpool_limits(1):
        t0 = time.perf_counter()
        A.training_call(*[np.asarray(a, np.float64) for a in arrs], [0, L],
                        A.Numerics(hadamard=hadamard, path="mixed" if path else "mxfp8", causal=causal))
        return time.perf_counter() - t0


def host_cpu():
    """(usable cores, CPU model) of this host."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    return n, model


def cpu_baseline(wl, causal: bool = True, max_len: int = CPU_SAMPLE_MAX_LEN):
    """The oracle, as it stands, on a bounded sample of the workload: every
    head of every document of at most ``max_len`` tokens (the first document
    if none is that short), one (document, head) per task over a pool of
    worker processes on the host's cores (at most CPU_WORKERS, the GPU's
    share of a box).  Run before the GPU is touched."""
    import multiprocessing as mp
    import numpy as np
    nproc, model = host_cpu()
    workers = max(1, min(CPU_WORKERS, nproc))
    g = wl.heads // wl.kv_heads
    docs = [i for i, L in enumerate(wl.doc_lens) if 0 < L <= max_len] or [0]
    tasks, flops = [], 0
    for i in docs:
        s, e = wl.cu_seqlens[i], wl.cu_seqlens[i + 1]
        L = e - s
        for hk in range(wl.kv_heads):
            qs = slice(hk * g, hk * g + g)
            arrs = [t[s:e][:, qs if t.shape[1] == wl.heads else slice(hk, hk + 1)].float().numpy()
                    for t in (wl.q, wl.k, wl.v, wl.do)]
            tasks.append((arrs, L, wl.hadamard, wl.path, causal))
            flops += 14 * wl.head_dim * g * (L * (L + 1) // 2 if causal else L * L)
    tasks.sort(key=lambda t: -t[1])            # longest first
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        cpu_s = sum(pool.map(_oracle_unit, tasks, chunksize=1))
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"all {wl.heads} heads of the {len(docs)} documents of at most {max_len} tokens "
                      f"({sum(wl.doc_lens[i] for i in docs)} tokens) of the {wl.name} workload: "
                      f"quantize+fwd+bwd of each (document, key/value head) unit, fp64 numpy, "
                      f"{workers} worker processes with single-threaded BLAS, {dt:.1f} s wall, {cpu_s:.1f} s CPU",
            "seconds": dt, "host_cores": nproc, "cpu_model": model, "flops": flops}


def measure(flamia, torch, wl, steps, warmup, causal_dq_scale=False, deterministic=False, exact=False,
            non_causal=False, exp2_fma=False):
    """Eager stage timing (HIP events between the entry points) over W + K
    steps, then the graph-replayed headline (median of 3 rounds of K)."""
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in (wl.q, wl.k, wl.v, wl.do))
    call = flamia.TrainingCall(q, k, v, do, wl.cu_seqlens, hadamard=wl.hadamard,
                               causal_dq_scale=wl.causal_dq_scale or causal_dq_scale, path=wl.path,
                               deterministic=deterministic, exact=exact, causal=not non_causal,
                               exp2_fma=exp2_fma)
    if non_causal:
        pairs = wl.heads * sum(L * L for L in wl.doc_lens)
    else:
        pairs = wl.causal_pairs()
    flops = 14 * wl.head_dim * pairs

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

    for _ in range(warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(steps):
        step(events[s_])
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / steps
    names = ["quantize", "attn_fwd", "bwd_prep", "attn_bwd", "bwd_finish"]
    stage_ms = {n: sum(ev[i].elapsed_time(ev[i + 1]) for ev in events) / steps for i, n in enumerate(names)}
    graph = graph_replay(call, torch, steps, warmup, flops)
    ms, timing = (graph["ms_per_step"], "hip_graph_replay") if "ms_per_step" in graph else (eager_ms, "eager")
    return dict(call=call, pairs=pairs, flops=flops, stage_ms=stage_ms, eager_ms=eager_ms, graph=graph,
                ms=ms, timing=timing)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="grouped-query variant of the workload: K and V with this many heads (0: one per query head)")
    ap.add_argument("--exact", action="store_true",
                    help="the exact option: per-token scales, all-tile V fold, per-row/per-key dS exponents")
    ap.add_argument("--non-causal", action="store_true",
                    help="the call without the causal mask (every key of a document visible); "
                         "FLOPs then count every (query, key) pair of a document")
    ap.add_argument("--causal-dq-scale", action="store_true",
                    help="the optional causal dQ accumulator scale (prescale from causally visible key blocks only)")
    ap.add_argument("--shape", default="",
                    help="one of the pages' packed benchmark shapes instead of --config: "
                         "equal_4x4096, equal_16x1024, equal_16x4096, equal_64x1024, "
                         "skew_8192_32x256, skew_8192_224x256")
    ap.add_argument("--exp2-fma", action="store_true",
                    help="exponentials of half of the 32x32 blocks on the FMA-pipe polynomial (both passes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the default run's extra measurements (config 4 both ways, the pages' equal and "
                         "skewed shapes, the 4-bit forward, exp2 on the FMA pipe)")
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

    wl = (workloads.pages_shape(args.shape, kv_heads=args.kv_heads) if args.shape
          else workloads.config(args.config, kv_heads=args.kv_heads))
    # the CPU baseline runs first, in forked workers, before anything touches the GPU
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, causal=not args.non_causal)

    flamia.load()
    m = measure(flamia, torch, wl, args.steps, args.warmup, args.causal_dq_scale, args.deterministic,
                args.exact, args.non_causal, args.exp2_fma)
    call, stage_ms, pairs, flops, ms_per_step = m["call"], m["stage_ms"], m["pairs"], m["flops"], m["ms"]
    if args.copy_calibration:
        dev = torch.device("cuda:0")
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    T, H, d = call.shape
    Hk = call.kv_heads
    grouped = Hk != H
    value = flops / (ms_per_step * 1e-3) / 1e12

    # roofline of the dominant kernel
    E, Ek = T * H * d, T * Hk * d
    # quantizer bytes: bf16 Q, K, V read; Q, K, V, per-key V codes written;
    # one exponent byte per token and head of Q and four planes of the K side
    qbytes = 3 * E + 7 * Ek + T * H + 4 * T * Hk
    plan_ms = plan_build_ms(flamia, torch, call)
    fwd_mix, bwd_mix = product_mix(d, pairs, bool(wl.path))
    kernels = {
        "attn_bwd": ("attn_bwd_kernel" if wl.path else "attn_bwd8_kernel", "mfma", 10 * d * pairs,
                     weighted_peak(bwd_mix)),
        "attn_fwd": ("attn_fwd_kernel", "mfma", 4 * d * pairs, weighted_peak(fwd_mix)),
        "quantize": ("quant_qkv_kernel", "hbm", qbytes, HBM_PEAK_GBS),
    }
    dom = max(kernels, key=lambda n: stage_ms[n])
    kname, bound, work, wpeak = kernels[dom]
    t_dom = stage_ms[dom] * 1e-3
    if bound == "mfma":
        achieved, unit, peak = work / t_dom / 1e12, "TFLOP/s", FP8_PEAK_TFLOPS
    else:
        achieved, unit, peak = work / t_dom / 1e9, "GB/s", HBM_PEAK_GBS
    traffic = (measured_traffic(kname, f"config{args.config}")
               if kname.startswith("attn_bwd") and not grouped and not args.exact and not args.non_causal
               and not args.deterministic and not args.causal_dq_scale
               else None)
    roofline = {"bound": bound, "kernel": kname, "achieved": achieved, "peak": peak, "unit": unit,
                "frac": achieved / peak, "traffic": traffic,
                "peak_note": ("MI355X dense FP8 matrix-core peak (every product counted at it)"
                              if bound == "mfma" else "HBM3E"),
                "frac_dtype_weighted": achieved / wpeak if bound == "mfma" else None,
                "dtype_weighted_peak": wpeak if bound == "mfma" else None,
                "algorithmic_work_per_launch": work, "avg_launch_ms": stage_ms[dom]}
    # the forward's own fraction of the FP8 peak (the other matrix-core kernel of the call)
    fname, _, fwork, fwpeak = kernels["attn_fwd"]
    f_ach = fwork / (stage_ms["attn_fwd"] * 1e-3) / 1e12
    roofline_fwd = {"bound": "mfma", "kernel": fname, "achieved": f_ach, "peak": FP8_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": f_ach / FP8_PEAK_TFLOPS,
                    "frac_dtype_weighted": f_ach / fwpeak, "dtype_weighted_peak": fwpeak,
                    "algorithmic_work_per_launch": fwork, "avg_launch_ms": stage_ms["attn_fwd"]}
    qk_ms = max(stage_ms["quantize"] - plan_ms, 1e-6)
    quant = {"quant_qkv_ms": qk_ms, "plan_ms": plan_ms, "launches": 3 if wl.path else 2,
             "GB/s": qbytes / (qk_ms * 1e-3) / 1e9,
             "frac_hbm_peak": qbytes / (qk_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
             "algorithmic_bytes": qbytes,
             "note": "quant_qkv_ms = quantize stage (HIP events) minus a separately timed work-list build"}

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": wl.name, "tokens": T, "heads": H, "kv_heads": Hk, "head_dim": d,
                   "doc_lens": wl.doc_lens if len(wl.doc_lens) <= 8 else f"{len(wl.doc_lens)} documents",
                   "hadamard": bool(wl.hadamard), "path": "mixed" if wl.path else "mxfp8",
                   "deterministic": bool(args.deterministic), "exact": bool(args.exact),
                   "exp2_fma": bool(args.exp2_fma),
                   "causal": not args.non_causal,
                   "causal_dq_scale": bool(wl.causal_dq_scale or args.causal_dq_scale),
                   "causal_pairs": pairs, "flops_per_step": flops},
        "pct_fp8_peak": 100.0 * value / FP8_PEAK_TFLOPS,
        "stage_ms": stage_ms, "event_ms_per_step": sum(stage_ms.values()),
        # the attention kernels alone: forward, and backward without the dO
        # quantization / D preparation (quantization excluded on both sides)
        "kernel_only_ms": {"fwd": stage_ms["attn_fwd"], "bwd": stage_ms["attn_bwd"] + stage_ms["bwd_finish"]},
        "quantizer": quant,
        "roofline": roofline,
        "roofline_fwd": roofline_fwd,
    }
    if not (wl.path or grouped or args.exact or args.deterministic or args.non_causal):
        # one untimed diagnostic backward on the state the timed steps left:
        # nonzero dS and those whose E4M3 code is zero
        counts = torch.zeros(2, dtype=torch.int64, device=call.dq.device)
        flamia.attn_bwd_main_diag(call.desc, call.qt, call.dk, call.dv, call.bws, None, 0, counts)
        nz, zero = (int(x) for x in counts.cpu())
        out["ds_zero_fraction"] = {"value": zero / max(nz, 1), "nonzero_ds": nz, "coded_zero": zero}
    out["toolchain"] = toolchain(torch)
    out["timing"] = m["timing"]
    out["eager_ms_per_step"] = m["eager_ms"]
    out["graph"] = m["graph"]
    del call, m
    if args.config == 3 and not args.no_extra and not (args.kv_heads or args.exact or args.non_causal
                                                       or args.deterministic or args.causal_dq_scale
                                                       or args.shape or args.exp2_fma):
        wl4 = workloads.config(4)
        extra = {"p4_forward": p4_forward_timing(flamia, torch, wl)}
        m4 = measure(flamia, torch, wl, args.steps, args.warmup, exp2_fma=True)
        extra["exp2_fma"] = {"workload": wl.name, "ms_per_step": m4["ms"],
                             "TFLOP/s": m4["flops"] / (m4["ms"] * 1e-3) / 1e12, "stage_ms": m4["stage_ms"],
                             "note": "exp2 of half of the 32x32 blocks on a degree-5 FMA-pipe polynomial, both passes"}
        del m4
        for tag, cds in (("long_context_32768", False), ("long_context_32768_causal_dq_scale", True)):
            m4 = measure(flamia, torch, wl4, args.steps, args.warmup, causal_dq_scale=cds)
            extra[tag] = {"workload": wl4.name, "causal_dq_scale": cds, "ms_per_step": m4["ms"],
                          "TFLOP/s": m4["flops"] / (m4["ms"] * 1e-3) / 1e12,
                          "pct_fp8_peak": 100.0 * m4["flops"] / (m4["ms"] * 1e-3) / 1e12 / FP8_PEAK_TFLOPS,
                          "timing": m4["timing"], "stage_ms": m4["stage_ms"], "flops_per_step": m4["flops"]}
            del m4
        for shape in ("equal_4x4096", "skew_8192_32x256", "skew_8192_224x256"):
            ws = workloads.pages_shape(shape)
            m4 = measure(flamia, torch, ws, args.steps, args.warmup)
            extra[shape] = {"workload": ws.name, "ms_per_step": m4["ms"],
                            "TFLOP/s": m4["flops"] / (m4["ms"] * 1e-3) / 1e12,
                            "pct_fp8_peak": 100.0 * m4["flops"] / (m4["ms"] * 1e-3) / 1e12 / FP8_PEAK_TFLOPS,
                            "stage_ms": m4["stage_ms"], "flops_per_step": m4["flops"]}
            del m4, ws
        out["extra"] = extra
    out["worklist"] = worklist_build(flamia, torch)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
