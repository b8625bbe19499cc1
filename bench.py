"""Benchmark of the exact-attention hot path on one MI355X.

A step is one pass of the whole path on one batch: fa_fwd (forward, O and LSE) then
fa_bwd (D = rowsum(dO*O), recompute, dQ/dK/dV) on the workload B=2, H=16, N=4096,
d=128, causal, bf16 inputs with Q scaled x4 (inputs drawn once with the seeded
generator and resident in HBM before timing). The metric is attention TFLOP/s under
the nominal count 4*B*H*N^2*d (halved when causal) for the forward pass plus 2.5x
that for the backward pass, against the dense bf16 matrix-core peak.

Prints ONE JSON line with the throughput, the roofline of the dominant kernel and of
the forward kernel (each kernel of the step timed with HIP events on the stream it runs
on: fa_bwd is run as its two stages, dQ with D and then dK/dV), per-pass median and
minimum times (from the timed steps, and from each pass run alone for at least 200 ms),
and the CPU oracle's throughput on a bounded sample of the same workload. The W warmup
steps are followed by WARM_S seconds of continuous work so that the timed steps run at
the sustained clock.

  python bench.py [--steps K (100)] [--warmup W (200)] [--gpus 1] [--sweep] [--split-kv] [--sparse]
                  [--dropout] [--deferred] [--configs] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 matrix peak (256 CU x 4096 FLOP/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0
WORKLOAD_ID = 4
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "counters_b2h16_n4096_d128_causal.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "io_aware_softmax_tiled_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` (a name prefix such as "bwd_dq_kernel") from the
    committed rocprofv3 counter runs, scaled by the copy-kernel calibration, or None when
    absent or taken on other kernel sources."""
    try:
        with open(PROFILE_COUNTERS) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    for name, k in rec.get("kernels", {}).items():
        if name.startswith(kernel) and "hbm_bytes_per_launch" in k:
            return k["hbm_bytes_per_launch"]
    return None


def cpu_baseline(inp, w, budget_heads=None):
    """Time the CPU oracle (as it stands) on a bounded sample of heads of the workload."""
    import oracle
    import workloads

    workers = oracle.attention.default_workers()
    nheads = budget_heads or min(w.B * w.H, max(2, workers))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)][:nheads]
    q, k, v, do = (workloads.as_f64(inp[n]) for n in ("q", "k", "v", "dout"))
    t0 = time.perf_counter()
    oracle.attention_forward_heads(q, k, v, w.scale, w.causal, None, heads=heads,
                                   workers=workers)
    oracle.attention_backward_heads(q, k, v, do, w.scale, w.causal, None, heads=heads,
                                    workers=workers)
    dt = time.perf_counter() - t0
    per_head = (w.fwd_flops() + w.bwd_flops()) / (w.B * w.H)
    return {
        "value": round(per_head * nheads / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": min(workers, nheads),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{nheads} of {w.B * w.H} heads of the same workload, forward + backward, "
                  f"float64 numpy, {dt:.1f} s wall",
    }


def pass_protocol(fa, torch, w, dev, ws, min_ms=200.0, min_calls=20):
    """Each pass on its own, called back to back until at least min_calls calls and
    min_ms of timed work, one HIP event pair per call on the stream the kernels run on:
    median and minimum per call. The forward pass is fa_fwd; the backward pass is the
    whole fa_bwd (both kernels), on O and LSE from a previous forward call."""
    stream = torch.cuda.current_stream()
    fwd = lambda: fa.fa_fwd(dev["q"], dev["k"], dev["v"], causal=w.causal, scale=w.scale,
                            out=dev["o"], lse=dev["lse"])
    fwd()
    bwd = lambda: fa.fa_bwd(dev["q"], dev["k"], dev["v"], dev["o"], dev["dout"], dev["lse"],
                            causal=w.causal, scale=w.scale, workspace=ws)
    out = {}
    for name, fn, flops in (("fwd", fwd, w.fwd_flops()), ("bwd", bwd, w.bwd_flops())):
        times, total = [], 0.0
        for _ in range(3):
            fn()
        while len(times) < min_calls or total < min_ms:
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(21)]
            evs[0].record(stream)
            for i in range(20):
                fn()
                evs[i + 1].record(stream)
            torch.cuda.synchronize()
            batch = [evs[i].elapsed_time(evs[i + 1]) for i in range(20)]
            times += batch
            total += sum(batch)
        med = statistics.median(times)
        out[name] = {"calls": len(times), "timed_ms": round(total, 2),
                     "median_ms": round(med, 4), "min_ms": round(min(times), 4),
                     "median_tflops": round(flops / (med * 1e-3) / 1e12, 2),
                     "median_pct_peak": round(100 * flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
    return out


# fa_bwd's kernels as fa_bwd_stage calls: stage 3 (dQ, forming and writing D), then
# stage 1 (dK/dV, reading D)
BWD_STAGES = (3, 1)


def run_step(fa, dev, w, ws, events=None):
    """fa_fwd, then fa_bwd as its stages (the same kernels fa_bwd launches, in the same
    order on the same stream), with events between the kernels when given."""
    rec = (lambda i: events[i].record()) if events is not None else (lambda i: None)
    o, lse = fa.fa_fwd(dev["q"], dev["k"], dev["v"], causal=w.causal, scale=w.scale,
                       out=dev["o"], lse=dev["lse"])
    rec(1)
    for i, stage in enumerate(BWD_STAGES):
        fa.fa_bwd_stage(stage, dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, dev["dq"],
                        dev["dk"], dev["dv"], ws, causal=w.causal, scale=w.scale)
        rec(2 + i)
    return dev["dq"]


# kernels of one step, in launch order, and the MFMA FLOPs each performs as a multiple
# of the nominal forward count (the forward: 2 products; dQ: S, dP, dQ; dK/dV: S, dP,
# dV, dK); at this workload (head_dim 128, no block mask or dropout) the dK/dV stage runs
# the two-wave kernel
KERNELS = [("fwd_kernel_16", 1.0), ("bwd_dq_kernel", 1.5), ("bwd_dkdv_pair_kernel", 2.0)]


# The GPU reaches its sustained clock only after tens of milliseconds of continuous
# work (measured: with 5 warmup steps the bench step ran at 607-611 TFLOP/s, after 50 or
# more at 686-694), and the inputs are drawn on the host first, so the device starts
# idle. Every timed region, the headline's included whatever --warmup is, is therefore
# preceded by WARM_S seconds of continuous work on the same shape.
WARM_S = 0.25


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bench_workload(fa, torch, w, inp, steps, warmup, warm_s=0.0):
    dev = {n: inp[n].cuda() for n in ("q", "k", "v", "dout")}
    dev["o"] = torch.empty(dev["q"].shape, dtype=torch.float32, device="cuda")
    dev["lse"] = torch.empty(dev["q"].shape[:3], dtype=torch.float32, device="cuda")
    for n in ("dq", "dk", "dv"):
        dev[n] = torch.empty(dev["q"].shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fa_bwd_workspace_size(w.B, w.H, w.N, w.d), dtype=torch.uint8,
                     device="cuda")
    for _ in range(warmup):
        run_step(fa, dev, w, ws)
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < warm_s:
        for _ in range(4):
            run_step(fa, dev, w, ws)
        torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(KERNELS) + 1)]
           for _ in range(steps)]
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record(stream)
        run_step(fa, dev, w, ws, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    samples = [[e[j].elapsed_time(e[j + 1]) for e in evs] for j in range(len(KERNELS))]
    per_kernel = [sum(x) / steps for x in samples]
    fwd_ms = per_kernel[0]
    bwd_ms = sum(per_kernel[1:])
    stats = {"kernels": [(statistics.median(x), min(x)) for x in samples],
             "fwd": (statistics.median(samples[0]), min(samples[0])),
             "bwd": (statistics.median([sum(t) for t in zip(*samples[1:])]),
                     min(sum(t) for t in zip(*samples[1:])))}
    return wall * 1e3 / steps, fwd_ms, bwd_ms, per_kernel, stats, dev, ws


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--sweep", action="store_true",
                    help="also print one line per sequence length (supplementary)")
    ap.add_argument("--split-kv", action="store_true",
                    help="also print split-KV lines: partial forward + merge against the "
                         "unsplit forward (supplementary)")
    ap.add_argument("--sparse", action="store_true",
                    help="also print block-sparse lines: forward and backward time against the "
                         "fraction of 128x128 blocks evaluated (supplementary)")
    ap.add_argument("--dropout", action="store_true",
                    help="also print dropout lines: forward and backward with the mask drawn "
                         "and regenerated on chip, against the kernels without dropout "
                         "(supplementary)")
    ap.add_argument("--deferred", action="store_true",
                    help="also print deferred-PV lines: the forward that keeps a query "
                         "block's whole numerator row on chip and multiplies by V once, "
                         "against the single-pass forward (supplementary)")
    ap.add_argument("--configs", action="store_true",
                    help="also print one line per parity workload (1-5): each pass's time, "
                         "TFLOP/s, % of peak and % of the roofline-attainable rate "
                         "(supplementary)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-workload", type=int, default=0, metavar="K",
                    help="only run parity workload K's passes (fa_fwd, then fa_bwd when the "
                         "workload has one), 10 untimed then 20 calls each: the program a "
                         "profiler wraps to take per-kernel counters on that workload")
    ap.add_argument("--summarize-profile", default="", metavar="DIR",
                    help="no GPU work: read the rocprofv3 kernel-trace and counter passes "
                         "under DIR (subfolders trace, fetch, write, sq, lds) and print a "
                         "JSON summary per kernel (time, HBM bytes scaled by the copy "
                         "calibration, MFMA busy, clock, LDS bank conflicts)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first copy a MIB-MiB buffer once (a plain copy kernel of known size, "
                         "to calibrate HBM byte counters in a profiler run)")
    args = ap.parse_args()
    if args.summarize_profile:
        print(json.dumps(summarize_profile(args.summarize_profile), indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (attention heads "
              "would shard across GPUs with no exchange between them).", file=sys.stderr)
        sys.exit(2)

    import torch

    import io_aware_softmax_tiled_amd as fa
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fa.load_library()
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.profile_workload:
        profile_workload(fa, torch, workloads, args.profile_workload)
        return
    w = workloads.WORKLOADS[WORKLOAD_ID]
    inp = workloads.draw(w)
    ms_step, fwd_ms, bwd_ms, per_kernel, stats, dev, ws = bench_workload(
        fa, torch, w, inp, args.steps, args.warmup, warm_s=WARM_S)
    protocol = pass_protocol(fa, torch, w, dev, ws)

    fwd_f, bwd_f = w.fwd_flops(), w.bwd_flops()
    value = (fwd_f + bwd_f) / (ms_step * 1e-3) / 1e12
    fwd_tf = fwd_f / (fwd_ms * 1e-3) / 1e12
    bwd_tf = bwd_f / (bwd_ms * 1e-3) / 1e12
    kernels = {}
    for (name, mult), ms, (med, mn) in zip(KERNELS, per_kernel, stats["kernels"]):
        kernels[name] = {"ms": round(ms, 4), "median_ms": round(med, 4), "min_ms": round(mn, 4)}
        if mult:
            kernels[name]["tflops"] = round(mult * fwd_f / (ms * 1e-3) / 1e12, 2)
    # the dominant kernel of the step: the longest average launch, timed live with HIP
    # events on the stream it runs on; achieved = its own MFMA FLOPs / its time
    dom = max(range(len(KERNELS)), key=lambda j: per_kernel[j])
    name, mult = KERNELS[dom]
    achieved = mult * fwd_f / (per_kernel[dom] * 1e-3) / 1e12
    roofline = {
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": measured_traffic(name),
        "kernel": name,
        "avg_launch_ms": round(per_kernel[dom], 4),
    }
    # the forward kernel's own roofline (the pass the 50%-of-peak target is set on)
    fwd_achieved = fwd_f / (per_kernel[0] * 1e-3) / 1e12
    roofline_fwd = {
        "bound": "mfma",
        "achieved": round(fwd_achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(fwd_achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": measured_traffic(KERNELS[0][0]),
        "kernel": KERNELS[0][0],
        "avg_launch_ms": round(per_kernel[0], 4),
    }
    line = {
        "metric": "attention fwd+bwd TFLOP/s (nominal 4BHN^2d/2 causal fwd + 2.5x bwd) and "
                  "% of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded i.i.d. N(0,1), Q x4)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "passes": "fwd+bwd"},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "warm_s": WARM_S,
        "passes": {"fwd": {"ms": round(fwd_ms, 4), "median_ms": round(stats["fwd"][0], 4),
                           "min_ms": round(stats["fwd"][1], 4), "tflops": round(fwd_tf, 2),
                           "pct_peak": round(100 * fwd_tf / PEAK_BF16_TFLOPS, 2)},
                   "bwd": {"ms": round(bwd_ms, 4), "median_ms": round(stats["bwd"][0], 4),
                           "min_ms": round(stats["bwd"][1], 4), "tflops": round(bwd_tf, 2),
                           "pct_peak": round(100 * bwd_tf / PEAK_BF16_TFLOPS, 2)}},
        "pass_protocol": protocol,
        "kernels": kernels,
        "roofline": roofline,
        "roofline_fwd": roofline_fwd,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(inp, w),
    }
    print(json.dumps(line), flush=True)

    if args.sweep:
        sweep(fa, torch, workloads)
    if args.split_kv:
        split_kv(fa, torch, workloads)
    if args.sparse:
        sparse(fa, torch, workloads)
    if args.dropout:
        dropout(fa, torch, workloads)
    if args.deferred:
        deferred(fa, torch, workloads)
    if args.configs:
        configs(fa, torch, workloads)


def sweep(fa, torch, workloads):
    """Supplementary lines: TFLOP/s vs sequence length at 16K tokens x 2048 hidden."""
    for d in (64, 128):
        for causal in (False, True):
            for N in (512, 1024, 2048, 4096, 8192, 16384):
                B, H = max(1, 16384 // N), 2048 // d
                w, inp = workloads.custom(B, H, N, d, "bf16", causal, seed=0)
                ms_step, fwd_ms, bwd_ms, *_ = bench_workload(fa, torch, w, inp, 10, 3,
                                                             warm_s=WARM_S)
                print(json.dumps({
                    "sweep": True, "B": B, "H": H, "N": N, "d": d, "causal": causal,
                    "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
                    "fwd_tflops": round(w.fwd_flops() / fwd_ms / 1e9, 2),
                    "bwd_tflops": round(w.bwd_flops() / bwd_ms / 1e9, 2)}), flush=True)


def _time(torch, fn, iters=20, warmup=3, warm_s=WARM_S):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < warm_s:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def split_kv(fa, torch, workloads):
    """Supplementary lines: fa_fwd_partial + fa_merge against fa_fwd on shapes with few
    query blocks per CU (where splitting the key axis adds workgroups) and on the
    benchmarked shape. Outputs are preallocated; the merge's HBM rate is its
    algorithmic bytes (n_splits*(d+1) floats read, d+1 written per row) over its time.
    After each shape's lines, one `split_hint` line compares the split fa_split_hint
    recommends (0: unsplit) with the fastest of the options timed, and times fa_fwd_auto
    (the same choice in one call, through a preallocated workspace)."""
    shapes = [(1, 4, 8192, 128, False), (1, 4, 8192, 128, True), (1, 2, 16384, 128, True),
              (1, 8, 4096, 128, True), (1, 8, 8192, 128, True), (1, 2, 8192, 64, False),
              (2, 2, 16384, 64, True), (1, 8, 16384, 64, False), (1, 4, 16384, 64, True),
              (1, 16, 2048, 128, False), (1, 8, 4096, 128, False), (1, 8, 8192, 128, False),
              (1, 16, 8192, 128, True),
              (2, 16, 4096, 128, True)]
    for B, H, N, d, causal in shapes:
        times = {}
        w, inp = workloads.custom(B, H, N, d, "bf16", causal, seed=0, with_dout=False)
        dev = {n: inp[n].cuda() for n in ("q", "k", "v")}
        o = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        t_full = _time(torch, lambda: fa.fa_fwd(dev["q"], dev["k"], dev["v"], causal=causal,
                                                scale=w.scale, out=o, lse=lse))
        for split_len in (N // 8, N // 4, N // 2):
            P = fa.fa_split_count(N, split_len)
            o_p = torch.empty((P, B, H, N, d), dtype=torch.float32, device="cuda")
            l_p = torch.empty((P, B, H, N), dtype=torch.float32, device="cuda")
            part = lambda: fa.fa_fwd_partial(dev["q"], dev["k"], dev["v"], split_len=split_len,
                                             causal=causal, scale=w.scale, out=o_p, lse=l_p)
            merge = lambda: fa.fa_merge(o_p, l_p, out=o, lse=lse)
            t_part = _time(torch, part)
            t_merge = _time(torch, merge)
            times[split_len] = t_part + t_merge
            merge_bytes = 4.0 * B * H * N * (P * (d + 1) + (d + 1))
            print(json.dumps({
                "split_kv": True, "B": B, "H": H, "N": N, "d": d, "causal": causal,
                "split_len": split_len, "n_splits": P,
                "unsplit_fwd_ms": round(t_full, 4), "partial_ms": round(t_part, 4),
                "merge_ms": round(t_merge, 4),
                "split_total_ms": round(t_part + t_merge, 4),
                "unsplit_tflops": round(w.fwd_flops() / t_full / 1e9, 2),
                "split_tflops": round(w.fwd_flops() / (t_part + t_merge) / 1e9, 2),
                "merge_hbm_gbs": round(merge_bytes / t_merge / 1e6, 1),
                "merge_hbm_frac": round(merge_bytes / t_merge / 1e6 / PEAK_HBM_GBS, 4)}),
                flush=True)
            del o_p, l_p
        hint = fa.fa_split_hint(B, H, N, d, causal=causal)
        times[0] = t_full
        best = min(times, key=times.get)
        ws_bytes = fa.fa_fwd_workspace_size(B, H, N, d, causal=causal)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
        t_auto = _time(torch, lambda: fa.fa_fwd_auto(dev["q"], dev["k"], dev["v"], causal=causal,
                                                     scale=w.scale, out=o, lse=lse, workspace=ws))
        print(json.dumps({
            "split_hint": True, "B": B, "H": H, "N": N, "d": d, "causal": causal,
            "hint_split_len": hint, "hint_ms": round(times.get(hint, float("nan")), 4),
            "auto_ms": round(t_auto, 4), "workspace_bytes": ws_bytes,
            "unsplit_ms": round(t_full, 4), "best_split_len": best,
            "best_ms": round(times[best], 4),
            "hint_over_best": round(times.get(hint, float("nan")) / times[best], 3)}),
            flush=True)
        del ws


def sparse(fa, torch, workloads):
    """Supplementary lines: block-sparse forward/backward time against the fraction of
    evaluated 128x128 blocks (random, diagonal blocks always on), next to the dense
    kernels on the same inputs. FLOPs are counted over the evaluated blocks only."""
    import numpy as np
    blk = fa.FA_SPARSE_BLOCK
    for B, H, N, d, causal in [(2, 16, 4096, 128, True), (1, 16, 8192, 64, False)]:
        w, inp = workloads.custom(B, H, N, d, "bf16", causal, seed=0)
        dev = {n: inp[n].cuda() for n in ("q", "k", "v", "dout")}
        nb = N // blk
        ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8,
                         device="cuda")
        o, lse = fa.fa_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=w.scale)
        t_fd = _time(torch, lambda: fa.fa_fwd(dev["q"], dev["k"], dev["v"], causal=causal,
                                              scale=w.scale, out=o, lse=lse))
        t_bd = _time(torch, lambda: fa.fa_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse,
                                              causal=causal, scale=w.scale, workspace=ws))
        full = np.tril(np.ones((nb, nb))) if causal else np.ones((nb, nb))
        for density in (1.0, 0.5, 0.25, 0.125):
            rng = np.random.default_rng(1)
            m = ((rng.random((nb, nb)) < density) * full).astype(np.uint8)
            np.fill_diagonal(m, 1)
            bm = torch.from_numpy(m).cuda()
            frac = float(m.sum() / full.sum())
            os_, ls_ = fa.fa_fwd_sparse(dev["q"], dev["k"], dev["v"], bm, causal=causal,
                                        scale=w.scale)
            t_f = _time(torch, lambda: fa.fa_fwd_sparse(dev["q"], dev["k"], dev["v"], bm,
                                                        causal=causal, scale=w.scale,
                                                        out=os_, lse=ls_))
            t_b = _time(torch, lambda: fa.fa_bwd_sparse(dev["q"], dev["k"], dev["v"], os_,
                                                        dev["dout"], ls_, bm, causal=causal,
                                                        scale=w.scale, workspace=ws))
            print(json.dumps({
                "sparse": True, "B": B, "H": H, "N": N, "d": d, "causal": causal,
                "block": blk, "blocks_on_frac": round(frac, 4),
                "dense_fwd_ms": round(t_fd, 4), "dense_bwd_ms": round(t_bd, 4),
                "sparse_fwd_ms": round(t_f, 4), "sparse_bwd_ms": round(t_b, 4),
                "fwd_time_frac": round(t_f / t_fd, 4), "bwd_time_frac": round(t_b / t_bd, 4),
                "sparse_fwd_tflops": round(frac * w.fwd_flops() / t_f / 1e9, 2),
                "sparse_bwd_tflops": round(frac * w.bwd_flops() / t_b / 1e9, 2)}), flush=True)



def dropout(fa, torch, workloads):
    """Supplementary lines: forward and backward with dropout (Philox blocks drawn in the
    forward kernel and drawn again in both backward kernels) next to the same kernels
    without dropout, on the same inputs. FLOPs are the dense nominal counts."""
    for B, H, N, d, causal in [(2, 16, 4096, 128, True), (1, 16, 8192, 64, False)]:
        w, inp = workloads.custom(B, H, N, d, "bf16", causal, seed=0)
        dev = {n: inp[n].cuda() for n in ("q", "k", "v", "dout")}
        ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8,
                         device="cuda")
        o, lse = fa.fa_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=w.scale)
        t_fd = _time(torch, lambda: fa.fa_fwd(dev["q"], dev["k"], dev["v"], causal=causal,
                                              scale=w.scale, out=o, lse=lse))
        t_bd = _time(torch, lambda: fa.fa_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse,
                                              causal=causal, scale=w.scale, workspace=ws))
        for p in (0.1,):
            kw = dict(p=p, seed=1234, offset=0, causal=causal, scale=w.scale)
            od, ld = fa.fa_fwd_dropout(dev["q"], dev["k"], dev["v"], **kw)
            t_f = _time(torch, lambda: fa.fa_fwd_dropout(dev["q"], dev["k"], dev["v"], out=od,
                                                         lse=ld, **kw))
            t_b = _time(torch, lambda: fa.fa_bwd_dropout(dev["q"], dev["k"], dev["v"], od,
                                                         dev["dout"], ld, workspace=ws, **kw))
            print(json.dumps({
                "dropout": True, "p": p, "B": B, "H": H, "N": N, "d": d, "causal": causal,
                "dense_fwd_ms": round(t_fd, 4), "dense_bwd_ms": round(t_bd, 4),
                "dropout_fwd_ms": round(t_f, 4), "dropout_bwd_ms": round(t_b, 4),
                "fwd_time_ratio": round(t_f / t_fd, 4), "bwd_time_ratio": round(t_b / t_bd, 4),
                "dropout_fwd_tflops": round(w.fwd_flops() / t_f / 1e9, 2),
                "dropout_bwd_tflops": round(w.bwd_flops() / t_b / 1e9, 2)}), flush=True)



def deferred(fa, torch, workloads):
    """Supplementary lines: the deferred-PV forward (numerator row kept on chip, one
    product with V) against the single-pass forward, on the BERT-large key-padding
    workload and on short sequences at 8K tokens. FLOPs are the nominal counts."""
    shapes = [(8, 16, 512, 64, False, (256, 512))]
    for N in (128, 256, 512):
        for d in (64, 128):
            for causal in (False, True):
                shapes.append((8192 // N, 2048 // d, N, d, causal, None))
    for B, H, N, d, causal, kv in shapes:
        w, inp = workloads.custom(B, H, N, d, "bf16", causal, kv_range=kv, seed=0,
                                  with_dout=False)
        dev = {n: inp[n].cuda() for n in ("q", "k", "v")}
        kvl = None if inp["kv_len"] is None else inp["kv_len"].cuda()
        o = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        kw = dict(causal=causal, scale=w.scale, kv_len=kvl, out=o, lse=lse)
        t_one = _time(torch, lambda: fa.fa_fwd(dev["q"], dev["k"], dev["v"], **kw))
        t_def = _time(torch, lambda: fa.fa_fwd_deferred(dev["q"], dev["k"], dev["v"], **kw))
        print(json.dumps({
            "deferred_pv": True, "B": B, "H": H, "N": N, "d": d, "causal": causal,
            "kv_range": kv, "single_pass_ms": round(t_one, 4), "deferred_ms": round(t_def, 4),
            "time_ratio": round(t_def / t_one, 4),
            "single_pass_tflops": round(w.fwd_flops() / t_one / 1e9, 2),
            "deferred_tflops": round(w.fwd_flops() / t_def / 1e9, 2)}), flush=True)



def profile_workload(fa, torch, workloads, wid, calls=20):
    """Parity workload wid's passes, a fixed number of calls each, for a profiler run."""
    w = workloads.WORKLOADS[wid]
    inp = workloads.draw(w)
    dev = {n: (None if inp[n] is None else inp[n].cuda()) for n in ("q", "k", "v", "dout")}
    kvl = None if inp["kv_len"] is None else inp["kv_len"].cuda()
    kw = dict(causal=w.causal, scale=w.scale, kv_len=kvl)
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fa_bwd_workspace_size(w.B, w.H, w.N, w.d), dtype=torch.uint8,
                     device="cuda")
    fns = [lambda: fa.fa_fwd(dev["q"], dev["k"], dev["v"], out=o, lse=lse, **kw)]
    if w.has_bwd:
        fns.append(lambda: fa.fa_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse,
                                     workspace=ws, **kw))
    for fn in fns:
        for _ in range(10 + calls):
            fn()
    torch.cuda.synchronize()
    print(json.dumps({"profiled_workload": wid, "name": w.name, "calls_per_pass": 10 + calls}),
          flush=True)


def _kernel_name(name):
    """Kernel template name without the namespace and the argument list."""
    import re
    n = re.sub(r"^void ", "", name).replace("fa::(anonymous namespace)::", "").replace("fa::", "")
    depth, out = 0, ""
    for ch in n:
        if ch == "(" and depth == 0:
            break
        depth += (ch == "<") - (ch == ">")
        out += ch
    return out.strip()


def summarize_profile(root, copy_mib=512):
    """Per-kernel summary of rocprofv3 outputs under root: kernel trace stats (trace/),
    FETCH_SIZE (fetch/), WRITE_SIZE, TCC_HIT, TCC_MISS (write/), SQ and GRBM counters
    (sq/), LDS counters (lds/). HBM bytes are the counters scaled so that a plain device
    copy of copy_mib MiB (launched first by --copy-calibration) reads and writes exactly
    its size."""
    import csv
    import glob

    def read_pass(sub):
        per = {}
        for f in glob.glob(os.path.join(root, sub, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for row in csv.DictReader(fh):
                    k = _kernel_name(row["Kernel_Name"])
                    did = row.get("Dispatch_Id") or row.get("Correlation_Id")
                    d = per.setdefault(k, {}).setdefault(row["Counter_Name"], {})
                    d[did] = d.get(did, 0.0) + float(row["Counter_Value"])
        return per

    def mean(per):
        return {k: {c: sum(v.values()) / len(v) for c, v in cs.items()} for k, cs in per.items()}

    raw = {p: read_pass(p) for p in ("fetch", "write", "sq", "lds")}
    passes = {p: mean(v) for p, v in raw.items()}

    def copy(p):
        # the calibration copy is the largest dispatch of any copy kernel in the pass (input
        # staging may launch the same copy kernel on smaller buffers)
        c = "FETCH_SIZE" if p == "fetch" else "WRITE_SIZE"
        return {c: max(max(v[c].values()) for k, v in raw[p].items()
                       if "copy" in k.lower() and c in v)}
    nbytes = copy_mib << 20
    try:
        fetch_factor = nbytes / (copy("fetch")["FETCH_SIZE"] * 1024)
        write_factor = nbytes / (copy("write")["WRITE_SIZE"] * 1024)
    except ValueError:  # no byte-counter passes (or no calibration copy in them)
        fetch_factor = write_factor = None
    trace = {}
    for f in glob.glob(os.path.join(root, "trace", "**", "*kernel_stats.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                trace[_kernel_name(row["Name"])] = row
    out = {"source_hash": kernel_source_hash(),
           "calibration": {"copy_mib": copy_mib, "fetch_factor": fetch_factor,
                           "write_factor": write_factor}, "kernels": {}}
    for k in passes["sq"]:
        if not any(k.startswith(p) for p in ("fwd_", "bwd_", "merge_")):
            continue
        s, l = passes["sq"][k], passes["lds"].get(k, {})
        fe, wr = passes["fetch"].get(k, {}), passes["write"].get(k, {})
        gui = s["GRBM_GUI_ACTIVE"] / 8
        e = {"calls": int(trace[k]["Calls"]) if k in trace else None,
             "trace_avg_us": float(trace[k]["AverageNs"]) / 1e3 if k in trace else None,
             "hbm_read_bytes": (fe["FETCH_SIZE"] * 1024 * fetch_factor
                                if fetch_factor and "FETCH_SIZE" in fe else None),
             "hbm_write_bytes": (wr["WRITE_SIZE"] * 1024 * write_factor
                                 if write_factor and "WRITE_SIZE" in wr else None),
             "l2_hit_rate": (wr["TCC_HIT"] / max(wr["TCC_HIT"] + wr["TCC_MISS"], 1.0)
                             if "TCC_HIT" in wr else None),
             "mfma_busy_frac": s["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * 1024),
             "mfma_insts": s["SQ_INSTS_MFMA"], "valu_insts": s["SQ_INSTS_VALU"],
             "lds_insts": l.get("SQ_INSTS_LDS"),
             "lds_bank_conflict_cycles": l.get("SQ_LDS_BANK_CONFLICT"),
             "lds_active_cycles": l.get("SQ_LDS_IDX_ACTIVE"),
             # LDS busy per compute unit; wave time waiting on LDS and issuing vector ALU
             # instructions (SQ cycle counters count quad-cycles, alike for both terms)
             "lds_active_frac": (l["SQ_LDS_IDX_ACTIVE"] / (256 * gui)
                                 if "SQ_LDS_IDX_ACTIVE" in l else None),
             "lds_wait_frac": (l["SQ_WAIT_INST_LDS"] / s["SQ_WAVE_CYCLES"]
                               if "SQ_WAIT_INST_LDS" in l else None),
             "valu_active_frac": (l["SQ_ACTIVE_INST_VALU"] / s["SQ_WAVE_CYCLES"]
                                  if "SQ_ACTIVE_INST_VALU" in l else None),
             "gui_active_cycles_per_xcd": gui}
        if e["hbm_read_bytes"] is not None and e["hbm_write_bytes"] is not None:
            e["hbm_bytes_per_launch"] = e["hbm_read_bytes"] + e["hbm_write_bytes"]
        if e["trace_avg_us"]:
            e["clock_ghz"] = gui / (e["trace_avg_us"] * 1e3)
        out["kernels"][k] = e
    return out


PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 matrix peak


def configs(fa, torch, workloads):
    """Supplementary lines: every parity workload timed on its own, with the roofline
    bound of each pass: attainable = min(peak, algorithmic FLOP/byte x 8 TB/s).
    Algorithmic bytes: forward Q, K, V in, O (fp32) and LSE out; backward Q, K, V, dO,
    O (fp32), LSE in, D written and read once, dQ, dK, dV (fp32) out."""
    for wid in sorted(workloads.WORKLOADS):
        w = workloads.WORKLOADS[wid]
        inp = workloads.draw(w)
        dev = {n: (None if inp[n] is None else inp[n].cuda()) for n in ("q", "k", "v", "dout")}
        kvl = None if inp["kv_len"] is None else inp["kv_len"].cuda()
        e = 4 if w.dtype == "f32" else 2
        bhn, bhnd = w.B * w.H * w.N, w.B * w.H * w.N * w.d
        peak = PEAK_F32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS
        kw = dict(causal=w.causal, scale=w.scale, kv_len=kvl)
        o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device="cuda")
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
        t_f = _time(torch, lambda: fa.fa_fwd(dev["q"], dev["k"], dev["v"], out=o, lse=lse, **kw))
        passes = [("fwd", t_f, w.fwd_flops(), 3 * bhnd * e + 4 * bhnd + 4 * bhn)]
        if w.has_bwd:
            ws = torch.empty(fa.fa_bwd_workspace_size(w.B, w.H, w.N, w.d), dtype=torch.uint8,
                             device="cuda")
            t_b = _time(torch, lambda: fa.fa_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse,
                                                 workspace=ws, **kw))
            passes.append(("bwd", t_b, w.bwd_flops(),
                           4 * bhnd * e + 4 * bhnd + 4 * bhn + 8 * bhn + 12 * bhnd))
        eff = None
        if inp["kv_len"] is not None:   # the work the kernels actually have to do
            eff = sum(4.0 * w.H * w.N * int(x) * w.d for x in inp["kv_len"].tolist())
        for name, t, flops, nbytes in passes:
            tf = flops / t / 1e9
            attain = min(peak, flops / nbytes * PEAK_HBM_GBS / 1e3)
            line = {"config": wid, "workload": w.name, "pass": name, "dtype": w.dtype,
                    "ms": round(t, 4), "tflops": round(tf, 2),
                    "pct_peak": round(100 * tf / peak, 2),
                    "bound": "mfma" if attain >= peak else "hbm",
                    "attainable_tflops": round(attain, 1),
                    "pct_attainable": round(100 * tf / attain, 2),
                    "algorithmic_mib": round(nbytes / 2**20, 1)}
            if eff is not None:
                mult = 1.0 if name == "fwd" else 2.5
                line["effective_tflops"] = round(mult * eff / t / 1e9, 2)
            print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
