#!/usr/bin/env python3
"""Benchmark of the W8A8 DiT linear on one MI355X.

A step is one pass of the hot path over one batch: per-token INT8 quantization of X
(qdt_quantize_per_token) followed by the INT8 MFMA GEMM with the fused dequant + bias
epilogue (qdt_w8a8_linear), on the 4608 x 4608 x 4608 attention projection (4096 image +
512 text tokens at hidden width 4608).  Weight preparation (calibration max-abs, smoothing,
weight quantization) is offline and untimed.  Inputs are seeded synthetic tensors resident
in HBM; R rotating buffer sets (each with its own X, Xq, Wq and Y) keep every step's
operands out of the 256 MB Infinity Cache.

Prints one JSON line: effective TOPS = 2 M N K / wall time per step, the GEMM's MFMA
roofline fraction (HIP events on the launch stream), the quantize pass's HBM fraction, the
CPU oracle timed on the host on the same workload, and the other workloads' timings.
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

METRIC = "W8A8 DiT linear effective TOPS at 4608³ (quant+GEMM+epilogue), % INT8 peak"
PEAK_INT8_TOPS = 5000.0    # MI355X dense INT8 MFMA
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_FP4_TOPS = 10100.0    # MI355X dense FP4 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the clock settles after about 20 ms of sustained load: the default warm-up covers ~45 ms
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="minimum warm-up load in milliseconds before the timed steps (the shader clock "
                         "settles under sustained MFMA load); the warm-up runs max(--warmup steps, this long)")
    ap.add_argument("--rotate", type=int, default=6, help="rotating buffer sets (cold Infinity Cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-run", action="store_true",
                    help="headline timing loop only (no step distribution, flushed steps, clock record or "
                         "accuracy pass): for runs under rocprofv3")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--only", default=None,
                    help="run only this workload's timing loop (per-workload profiles); the headline "
                         "workload skips the others and the CPU baseline, another prints its own line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain device copy of known size (HBM counter calibration)")
    ap.add_argument("--counters-from", default=None, metavar="DIR",
                    help="print a markdown summary (per kernel: dispatches, duration, counter means, MFMA busy "
                         "cycles per SIMD) of the rocprofv3 --pmc --kernel-trace CSVs under DIR and exit")
    ap.add_argument("--trace-from", default=None, metavar="DIR",
                    help="print a markdown summary of a rocprofv3 --kernel-trace run under DIR (per kernel, over "
                         "the later half of its dispatches: count, mean, median, min, max in microseconds) and exit")
    ap.add_argument("--traffic-from", default=None, metavar="DIR",
                    help="write profiles/*_traffic.json from rocprofv3 --pmc CSVs under DIR/{fetch,write,"
                         "copy_fetch,copy_write} and exit")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def to_dev(a):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


EVENT_EVERY = 10   # steps between event-bracketed steps (a timing event record costs ~5 us of stream time)
MIN_EVENT_PAIRS = 10


class _NoEvent:
    """Stands in for an event a sampled step does not record."""

    def record(self, *a, **k):
        pass


def warm_up(fn_step, sets, warmup, settle_ms=0.0):
    """`warmup` untimed steps, continued until at least `settle_ms` of wall time has passed.
    Returns the number of warm-up steps run."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while n < warmup or (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(50 if n >= warmup else min(50, warmup - n)):
            fn_step(sets[n % len(sets)], None)
            n += 1
        torch.cuda.synchronize()
    return n


def time_loop(fn_step, sets, steps, warmup, settle_ms=0.0, stats_out=None, clock_grid=None):
    """Wall time of `steps` steps (sync on both sides) + per-phase HIP event times.

    A step calls ev[0].record() before its first launch, ev[1].record() between its two launches
    and ev[2].record() after the second.  Every EVENT_EVERY-th step of the timed region is sampled,
    never more often: an event record costs the stream a few microseconds, and sampling every step
    of a short region (20 steps) measured 97.7 us per step against 86.1 for the same kernels
    sampled every 10th step.  When the timed region holds fewer than MIN_EVENT_PAIRS pairs, the
    steps and the sampling schedule continue right after it (untimed, same rotating sets and
    spacing, clock still settled) until it does.  The samples alternate: the first of a pair records ev[0] and ev[1] (phase 1 alone), the second
    ev[0] and ev[2] only, so that no event sits between the two launches of the step whose second
    phase is measured (an event record between two kernels delays the second one's start).  Phase
    2 of a pair is the second sample's interval minus the first's; an event interval's own fixed
    overhead cancels in that difference.  The other steps run without events.  With `clock_grid`
    (the GEMM's workgroup count) the library's clock record is armed over the timed steps, and the
    GEMM's shader clock during them goes to stats_out["clock"]."""
    import torch
    # Everything the timed region needs is allocated before the warm-up: an allocation between the
    # warm-up and the timed steps leaves the GPU idle for a few milliseconds, after which its clock
    # takes ~40 ms of load to come back (measured: the first 400 steps after such a gap ran 7-9%
    # slower), which is longer than the timed region.
    every = EVENT_EVERY
    # the sampling schedule runs on past the timed region (same spacing) until it holds
    # MIN_EVENT_PAIRS pairs; denser sampling after the region measured the GEMM 8% faster than in it
    total = max(steps, 2 * MIN_EVENT_PAIRS * every)
    sampled = list(range(0, total, every))
    sampled = sampled[: len(sampled) // 2 * 2]
    n_in = sum(1 for i in sampled if i < steps)
    none = _NoEvent()
    evs = {}
    for n, i in enumerate(sampled):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        evs[i] = [e[0], e[1], none] if n % 2 == 0 else [e[0], none, e[2]]
    rec = None
    if clock_grid is not None:
        import quantized_diffusion_transformer_amd as qdt
        rec = torch.zeros((steps * clock_grid, 4), dtype=torch.int64, device="cuda")
    nw = warm_up(fn_step, sets, warmup, settle_ms)
    if stats_out is not None:
        stats_out["warmup_steps_run"] = nw
    if rec is not None:
        qdt.clock_record(rec)  # host-side arming only
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn_step(sets[i % len(sets)], evs.get(i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if rec is not None:
        used = qdt.clock_record_used()
        qdt.clock_record(None)
        if stats_out is not None:
            stats_out["clock"] = clock_stats(rec[:used], clock_grid)
    for i in range(steps, total):
        fn_step(sets[i % len(sets)], evs.get(i))
    torch.cuda.synchronize()
    if stats_out is not None:
        stats_out["event_every"] = every
        stats_out["event_samples"] = len(sampled)
        stats_out["event_samples_in_timed_region"] = n_in
        stats_out["event_samples_after_timed_region"] = len(sampled) - n_in
        stats_out["event_pairs"] = len(sampled) // 2
    ph1 = [evs[i][0].elapsed_time(evs[i][1]) for i in sampled[0::2]]
    both = [evs[i][0].elapsed_time(evs[i][2]) for i in sampled[1::2]]
    ph2 = [b - a for a, b in zip(ph1, both)]
    return (t1 - t0) * 1e3 / steps, ph1, ph2


def step_distribution(fn_step, sets, blocks=30, per_block=10):
    """Mean step time of each of `blocks` runs of `per_block` back-to-back steps, bracketed by HIP
    events at the block ends only (the event cost is spread over the block)."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(blocks + 1)]
    n = 0
    evs[0].record()
    for b in range(blocks):
        for _ in range(per_block):
            fn_step(sets[n % len(sets)], None)
            n += 1
        evs[b + 1].record()
    torch.cuda.synchronize()
    return [evs[b].elapsed_time(evs[b + 1]) / per_block for b in range(blocks)]


FLUSH_BYTES = 512 << 20  # more than the 256 MB Infinity Cache


def flushed_steps(fn_step, sets, reps=25):
    """Single steps bracketed by HIP events, each after a 512 MiB write that evicts the caches
    (outside the events)."""
    import torch
    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    times = []
    for r in range(reps):
        scratch.fill_(r & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn_step(sets[r % len(sets)], None)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del scratch
    return times


def clock_stats(buf, grid):
    """Shader clock of the GEMM kernel from the library's clock record: per launch, the sum over
    workgroups of shader-clock cycles over the sum of 100 MHz real-time ticks, from each
    workgroup's start to its last store; median and p10 / p90 over the launches."""
    import numpy as np
    rec = buf.cpu().numpy().astype(np.int64).reshape(-1, grid, 4)
    cyc = (rec[:, :, 2] - rec[:, :, 0]).sum(axis=1).astype(np.float64)
    real = (rec[:, :, 3] - rec[:, :, 1]).sum(axis=1).astype(np.float64)
    mhz = cyc / real * 100.0
    span_us = (rec[:, :, 3].max(axis=1) - rec[:, :, 1].min(axis=1)) / 100.0
    return {"clock_mhz": float(np.median(mhz)), "clock_mhz_p10": float(np.percentile(mhz, 10)),
            "clock_mhz_p90": float(np.percentile(mhz, 90)), "launches": int(rec.shape[0]),
            "kernel_span_us_median": float(np.median(span_us)),
            "how": "over the timed steps: s_memtime / s_memrealtime read by each workgroup's first wave at its "
                   "start and after its last store; clock = sum of cycles / sum of 100 MHz ticks per launch "
                   "(median over launches)"}


def time_loop_best(fn_step, steps, warmup, reps=2, clock_grid=None, info=None):
    """time_loop on one buffer set, repeated: the repetition with the lowest wall time (context
    numbers of the other workloads; a one-off stall of the device then costs a repetition, not
    the number).  With clock_grid, info["clock"] is the GEMM clock over that repetition."""
    best = None
    for r in range(reps):
        st = {}
        res = time_loop(fn_step, [None], steps, warmup if r == 0 else max(1, warmup // 4),
                        settle_ms=100.0 if r == 0 else 0.0, stats_out=st, clock_grid=clock_grid)
        if best is None or res[0] < best[0]:
            best = res
            if info is not None and "clock" in st:
                info["clock"] = st["clock"]
    return best


def stats(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return dict(mean=float(a.mean()), median=float(np.median(a)), p10=float(np.percentile(a, 10)),
                p90=float(np.percentile(a, 90)))


def traffic_record(name):
    """HBM bytes per launch measured with rocprofv3 counters, valid only for the kernel source it
    was taken on (null once the source changed)."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = open(os.path.join(ROOT, "quantized_diffusion_transformer_amd", "csrc", rec["source"]), "rb").read()
    if hashlib.sha256(src).hexdigest() != rec["source_sha256"]:
        return None
    return rec


# ---------------------------------------------------------------- HBM traffic from counters
COPY_BYTES = 256 << 20  # plain copy of 256 MiB: reads and writes this many bytes
TRAFFIC_KERNELS = {  # record name -> (kernel-name substring, source file the record is valid for)
    "w8a8_gemm_bias_4608": ("gemm_kernel", "qdt_gemm.hip"),
    "quantize_4608": ("quant_rows_kernel", "qdt_quant.hip"),
}


def calibrate_copy():
    """A plain device-to-device copy of COPY_BYTES, a few times, for FETCH_SIZE / WRITE_SIZE scaling."""
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 5}), flush=True)


def _pmc_means(d, counter):
    """Mean counter value (KiB per dispatch) per kernel name in the counter CSV under d."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    acc = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def write_traffic(d):
    """profiles/<name>_traffic.json: HBM bytes per launch = counter KiB x 1024 x (copy bytes / copy
    counter bytes), per direction, for the dominant kernels of the headline run."""
    res = {}
    scale = {}
    for direction, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        copy = _pmc_means(os.path.join(d, f"copy_{direction}"), counter)
        big = max(copy.values())  # the copy kernel is the largest dispatch of the calibration run
        scale[direction] = COPY_BYTES / (big * 1024.0)
        means = _pmc_means(os.path.join(d, direction), counter)
        for rec, (sub, _) in TRAFFIC_KERNELS.items():
            vals = [v for k, v in means.items() if sub in k]
            if vals:
                res.setdefault(rec, {})[direction] = max(vals) * 1024.0 * scale[direction]
    for rec, (sub, src) in TRAFFIC_KERNELS.items():
        if rec not in res or len(res[rec]) != 2:
            continue
        code = open(os.path.join(ROOT, "quantized_diffusion_transformer_amd", "csrc", src), "rb").read()
        out = {"kernel": sub, "source": src, "source_sha256": hashlib.sha256(code).hexdigest(),
               "fetch_bytes_per_launch": round(res[rec]["fetch"]), "write_bytes_per_launch": round(res[rec]["write"]),
               "bytes_per_launch": round(res[rec]["fetch"] + res[rec]["write"]),
               "copy_scale": {k: round(v, 5) for k, v in scale.items()}}
        with open(os.path.join(ROOT, "profiles", f"{rec}_traffic.json"), "w") as f:
            json.dump(out, f, indent=1)
        print(json.dumps({rec: out}), flush=True)


N_SIMD = 1024  # MI355X: 256 CUs x 4 SIMDs


def summarize_trace(d, last_fraction=0.5):
    """Per-kernel duration statistics of a rocprofv3 kernel trace, over the later `last_fraction` of
    each kernel's dispatches (the timed steps follow the warm-up)."""
    import csv
    import glob
    import numpy as np
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no kernel_trace.csv under {d}")
    durs = {}
    for f in files:
        rows = sorted(csv.DictReader(open(f)), key=lambda r: int(r["Start_Timestamp"]))
        for r in rows:
            durs.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["| kernel | dispatches (all) | summarized | mean | median | min | max |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for k, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        w = np.asarray(v[int(len(v) * (1 - last_fraction)):] if len(v) >= 4 else v)
        lines.append(f"| `{k[:100]}` | {len(v)} | {len(w)} | {w.mean():.2f} | {np.median(w):.2f} | {w.min():.2f} | "
                     f"{w.max():.2f} |")
    print("\n".join(lines), flush=True)


def summarize_counters(d, last_fraction=0.5):
    """Markdown table per kernel of a rocprofv3 counter run (its later dispatches: the timed steps):
    dispatches, mean duration, mean of each counter (rocprofv3 sums over XCDs, shader engines and
    SIMDs), and SQ_VALU_MFMA_BUSY_CYCLES per SIMD."""
    import csv
    import glob
    cc = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not cc:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    per, name, dur = {}, {}, {}
    for f in cc:
        for r in csv.DictReader(open(f)):
            k = (f, int(r["Dispatch_Id"]))
            per.setdefault(k, {})[r["Counter_Name"]] = float(r["Counter_Value"])
            name[k] = r["Kernel_Name"]
            dur[k] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    byk = {}
    for k in sorted(per):
        byk.setdefault(name[k], []).append(k)
    lines = []
    for kn, ks in byk.items():
        ks = ks[int(len(ks) * (1 - last_fraction)):] if len(ks) >= 4 else ks
        cnames = sorted(per[ks[0]])
        mean = {c: sum(per[k][c] for k in ks) / len(ks) for c in cnames}
        us = sum(dur[k] for k in ks) / len(ks) / 1e3
        lines.append(f"### `{kn[:110]}`")
        lines.append("")
        lines.append(f"{len(ks)} dispatches, mean duration {us:.2f} us")
        lines.append("")
        lines.append("| counter | mean per dispatch |")
        lines.append("|---|---:|")
        for c in cnames:
            lines.append(f"| {c} | {mean[c]:.5g} |")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            lines.append(f"| SQ_VALU_MFMA_BUSY_CYCLES per SIMD | {mean['SQ_VALU_MFMA_BUSY_CYCLES'] / N_SIMD:.5g} |")
        lines.append("")
    print("\n".join(lines), flush=True)


def headline(args):
    import numpy as np
    import torch

    import qdt_workloads as W
    import quantized_diffusion_transformer_amd as qdt

    name = W.HEADLINE
    log(f"generating {name}")
    d = W.make_workload(name)
    M, N, K = d["M"], d["N"], d["K"]
    X0, W0, b = to_dev(d["X"]), to_dev(d["W"]), to_dev(d["bias"])
    s = qdt.channel_absmax(X0)
    Wq0, sw, inv, lam = qdt.smooth_prepare(W0, s)
    torch.cuda.synchronize()
    plan = qdt.linear_plan(M, N, K, "bias")
    R = max(1, args.rotate)
    sets = []
    for r in range(R):
        X = X0 if r == 0 else X0.clone()
        Wq = Wq0 if r == 0 else Wq0.clone()
        sets.append(dict(X=X, Wq=Wq, Xq=torch.empty((M, K), dtype=torch.int8, device="cuda"),
                         sx=torch.empty(M, dtype=torch.float32, device="cuda"),
                         Y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))
    torch.cuda.synchronize()

    def step(S, ev):
        if ev is not None:
            ev[0].record()
        qdt.quantize_per_token(S["X"], inv, S["Xq"], S["sx"])
        if ev is not None:
            ev[1].record()
        qdt.w8a8_linear(S["Xq"], S["sx"], S["Wq"], sw, b, "bias", out=S["Y"])
        if ev is not None:
            ev[2].record()

    log(f"timing {args.steps} steps (warmup {args.warmup} steps and >= {args.settle_ms} ms, {R} rotating sets), "
        f"plan {plan}")
    info = {}
    ms, tq, tg = time_loop(step, sets, args.steps, args.warmup, args.settle_ms, info, clock_grid=plan["grid"])
    log(f"wall {ms:.4f} ms/step; quantize {stats(tq)['mean']:.4f} ms + linear {stats(tg)['mean']:.4f} ms (HIP events)")
    clk = info["clock"]
    if args.profile_run:
        dist, flushed, acc, protocols, vendor = [ms], [ms], None, None, None
    else:
        dist = step_distribution(step, sets)
        flushed = flushed_steps(step, sets)
        log(f"step blocks median {np.median(dist):.4f} ms; flushed median {np.median(flushed):.4f} ms; "
            f"GEMM clock {clk['clock_mhz']:.0f} MHz")
        acc = accuracy_info(d, sets[0]["Y"], W0, b, qdt)
        protocols = protocol_variants(step, sets, plan, M * N * K * 2.0)
        vendor = vendor_reference(sets[0], sw, qdt)
    del W0
    ops = 2.0 * M * N * K
    tops = ops / (ms * 1e-3) / 1e12
    q = stats(tq)
    g = stats(tg)
    qbytes = 2 * M * K + M * K + 4 * M + 4 * K
    gbytes = M * K + N * K + 4 * M + 4 * N + 2 * N + 2 * M * N
    gemm_tops = ops / (g["mean"] * 1e-3) / 1e12
    traffic = traffic_record("w8a8_gemm_bias_4608")
    peak_clk = PEAK_INT8_TOPS * clk["clock_mhz"] / 2400.0
    out = {
        "metric": METRIC,
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "warmup_steps_run": info["warmup_steps_run"],
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": name, "M": M, "N": N, "K": K, "epilogue": "bias", "smoothquant_alpha": 0.5,
                   "plan": plan, "rotating_sets": R},
        "pct_int8_peak": round(100.0 * tops / PEAK_INT8_TOPS, 2),
        "step_ms": {"back_to_back_blocks": {k: round(v, 5) for k, v in stats(dist).items()},
                    "blocks": len(dist), "steps_per_block": 10,
                    "flushed_single": {k: round(v, 5) for k, v in stats(flushed).items()}, "flushed_reps": len(flushed),
                    "note": "back_to_back_blocks: mean step of each block of 10 rotating-set steps (HIP events at "
                            "block ends); flushed_single: one step between HIP events after a 512 MiB write that "
                            "evicts L2 and the Infinity Cache (includes the event-to-launch gap)"},
        "clock_mhz": round(clk["clock_mhz"], 1),
        "clock": {k: (round(v, 2) if isinstance(v, float) else v) for k, v in clk.items()},
        "roofline": {"bound": "mfma", "kernel": "gemm_kernel (qdt_w8a8_linear, BIAS)",
                     "achieved": round(gemm_tops, 2), "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                     "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
                     "traffic": None if traffic is None else traffic["bytes_per_launch"],
                     "algorithmic_ops_per_launch": ops, "avg_launch_ms": round(g["mean"], 5),
                     "launch_ms": {k: round(v, 5) for k, v in g.items()},
                     "event_samples": info["event_samples"],
                     "event_samples_in_timed_region": info["event_samples_in_timed_region"],
                     "event_samples_after_timed_region": info["event_samples_after_timed_region"],
                     "timing": "HIP events on the library's stream, in pairs of sampled steps: (quantize + "
                               "linear, no event between them) minus (quantize alone); every 10th step is sampled, "
                               "and when the timed region holds fewer than 10 pairs the steps and the schedule "
                               "continue after it until it does; the clock record's first-start-to-last-end span of the timed launches is "
                               "clock.kernel_span_us_median",
                     "peak_at_measured_clock": round(peak_clk, 1),
                     "frac_at_measured_clock": round(gemm_tops / peak_clk, 4)},
        "roofline_quantize": {"bound": "hbm", "kernel": "quant_rows_kernel (qdt_quantize_per_token)",
                              "achieved": round(qbytes / (q["mean"] * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                              "unit": "GB/s", "frac": round(qbytes / (q["mean"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                              "algorithmic_bytes_per_launch": qbytes, "avg_launch_ms": round(q["mean"], 5),
                              "launch_ms": {k: round(v, 5) for k, v in q.items()},
                              "timing": "HIP event interval, which also holds the dispatch gap between the event "
                                        "record and the kernel start; the kernel's own duration is in the "
                                        "rocprofv3 kernel trace",
                              "traffic": None if traffic_record("quantize_4608") is None
                              else traffic_record("quantize_4608")["bytes_per_launch"]},
        "accuracy_vs_fp64_unquantized": acc,
        "cache_protocols": protocols,
        "vendor_reference": vendor,
        "gemm_algorithmic_bytes": gbytes,
        "device": torch.cuda.get_device_name(0),
    }
    return out, d


def protocol_variants(step, sets, plan, ops):
    """Context for `value` (which rotates X and the weights through all sets, so both are read
    from HBM every step): the same step with only the weights rotating (X stays in the Infinity
    Cache, as when the previous kernel has just written it) and with one set (everything warm).
    Step time, effective TOPS, the GEMM's event time and its shader clock for each."""
    out = {}
    variants = (("rotate_weights_only", [dict(S, X=sets[0]["X"]) for S in sets]), ("single_set", [sets[0]]))
    for label, vs in variants:
        info = {}
        ms, _, tg = time_loop(step, vs, 200, 20, 150.0, info, clock_grid=plan["grid"])
        g = stats(tg)
        out[label] = {"sets": len(vs), "ms_per_step": round(ms, 5), "eff_tops": round(ops / (ms * 1e-3) / 1e12, 1),
                      "gemm_ms": round(g["mean"], 5), "gemm_tops": round(ops / (g["mean"] * 1e-3) / 1e12, 1),
                      "gemm_clock_mhz": round(info["clock"]["clock_mhz"], 1)}
        log(f"protocol {label}: {ms:.4f} ms/step, GEMM {g['mean']:.4f} ms at {info['clock']['clock_mhz']:.0f} MHz")
    return out


def vendor_reference(S, sw, qdt):
    """Context: the vendor BLAS's int8 GEMM (torch._int_mm, int8 x int8 -> int32) on the same
    quantized operands, warm, against this library's int32 accumulators (ACC_I32 epilogue) on the
    same data.  Neither is part of the timed path."""
    import torch
    try:
        Xq, Wq = S["Xq"], S["Wq"]
        M, K = Xq.shape
        N = Wq.shape[0]
        Bt = Wq.t()
        ref = torch._int_mm(Xq, Bt)
        own = qdt.w8a8_linear(Xq, S["sx"], Wq, sw, None, "acc_i32")
        torch.cuda.synchronize()

        def timed(fn, n=200):
            t_end = time.perf_counter() + 0.15
            while time.perf_counter() < t_end:
                fn()
                torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n
        ms_v = timed(lambda: torch._int_mm(Xq, Bt))
        ms_o = timed(lambda: qdt.w8a8_linear(Xq, S["sx"], Wq, sw, None, "acc_i32", out=own))
        ops = 2.0 * M * N * K
        return {"kernel": "torch._int_mm (int8 x int8 -> int32, the ROCm BLAS)", "ms": round(ms_v, 5),
                "tops": round(ops / (ms_v * 1e-3) / 1e12, 1),
                "own_acc_i32_ms": round(ms_o, 5), "own_acc_i32_tops": round(ops / (ms_o * 1e-3) / 1e12, 1),
                "int32_results_equal": bool(torch.equal(ref, own)),
                "note": "one warm operand set, 200 back-to-back launches between two HIP events"}
    except Exception as e:  # context only: a missing or failing library kernel does not end the run
        return {"kernel": "torch._int_mm", "error": repr(e)[:200]}


def accuracy_info(d, Y, Wt, b, qdt, nrows=64):
    """Information, not a gate: the W8A8 output's error against the unquantized linear in fp64
    (X W^T + b on the bf16 inputs) on sampled rows, with SmoothQuant (the timed path's output) and
    without smoothing (lambda = 1, run here once)."""
    import numpy as np
    import torch

    import qdt_workloads as W
    X = to_dev(d["X"])
    Wq, sw, _, _ = qdt.smooth_prepare(Wt, None)
    Xq, sx = qdt.quantize_per_token(X, None)
    Yp = qdt.w8a8_linear(Xq, sx, Wq, sw, b, "bias")
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(1).choice(d["M"], nrows, replace=False))
    ref = W.bf16_bits_to_f32(d["X"][rows]).astype(np.float64) @ W.bf16_bits_to_f32(d["W"]).astype(np.float64).T
    ref += W.bf16_bits_to_f32(d["bias"]).astype(np.float64)[None, :]
    out = {"rows": int(nrows)}
    for label, t in (("smoothquant_alpha_0.5", Y), ("no_smoothing", Yp)):
        y = t[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
        e = y - ref
        out[label] = {"rel_frobenius": round(float(np.linalg.norm(e) / np.linalg.norm(ref)), 6),
                      "max_abs": round(float(np.abs(e).max()), 6)}
    return out


def cpu_baseline(d):
    import numpy as np

    import oracle
    n = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    oracle.set_threads(min(n, os.cpu_count() or n))
    s = oracle.channel_absmax(d["X"])
    Wq, sw, inv, _ = oracle.smooth_prepare(d["W"], s)
    M, N, K = d["M"], d["N"], d["K"]
    # warm-up on a few rows, then whole linears (quantize + int32 GEMM + epilogue) until about
    # 10 s of wall time have passed
    oracle.linear_rows(*oracle.quantize_per_token(d["X"][:8], inv), Wq, sw, d["bias"], np.arange(8), "bias")
    n = 0
    t0 = time.perf_counter()
    while True:
        Xq, sx = oracle.quantize_per_token(d["X"], inv)
        acc = oracle.gemm_i32(Xq, Wq)
        oracle.epilogue(acc, sx, sw, d["bias"], "bias")
        n += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0:
            break
    return {"value": round(2.0 * M * N * K * n / dt / 1e12, 4), "unit": "TOPS", "cores": oracle.threads(),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"the whole {M}x{N}x{K} linear (quantize + int32 GEMM + BIAS epilogue) {n} times, "
                      f"after a warm-up on 8 rows"}


EXTRA_WORKLOADS = ("dit_ffn_gate_up_4608x24576x4608", "text_cond_proj_512x4608x53248",
                   "text_cond_proj_padded_4608x4608x53248", "qk_proj_headnorm_16896x4608x4608",
                   "qk_proj_headnorm_6037x4608x4608", "adaln_quantize_4608x4608", "adaln_quantize_16896x4608",
                   "mxfp4_attn_proj_4608x4608x4608", "mxfp4_ffn_gate_up_4608x24576x4608",
                   "mxfp4_qk_proj_headnorm_16896x4608x4608", "mxfp4_text_cond_proj_512x4608x53248",
                   "wo4_text_cond_proj_512x4608x53248", "wo8_text_cond_proj_512x4608x53248",
                   "attention_4608x18x256", "attention_16896x18x256")


def extra_workloads(args, only=None):
    """Timings of the other workloads (one rotating set; context for the other epilogues).
    ``only`` restricts the run to one of EXTRA_WORKLOADS (for per-workload profiles)."""
    import torch

    import qdt_workloads as W
    import quantized_diffusion_transformer_amd as qdt
    res = {}
    min_steps = max(5, args.steps // 5)

    def counts(step):
        """Warm-up of at least 50 ms of load (the clock settles after about 20 ms) and at least
        20 ms of timed steps, from the duration of a few untimed steps."""
        for _ in range(3):
            step(None, None)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(5):
            step(None, None)
        torch.cuda.synchronize()
        t = (time.perf_counter() - t0) / 5
        return max(min_steps, int(0.020 / t) + 1), max(20, int(0.050 / t) + 1)

    def prep(name, padded=False):
        d = W.make_workload(name, padded=padded)
        X, Wt = to_dev(d["X"]), to_dev(d["W"])
        s = qdt.channel_absmax(X)
        Wq, sw, inv, _ = qdt.smooth_prepare(Wt, s)
        torch.cuda.synchronize()
        return d, X, Wq, sw, inv

    def run(name, d, X, Wq, sw, inv, epi, extra=None, **kw):
        M, N, K = d["M"], d["N"], d["K"]
        Xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
        sx = torch.empty(M, dtype=torch.float32, device="cuda")
        b = None if d.get("bias") is None else to_dev(d["bias"])
        plan = qdt.linear_plan(M, N, K, epi)
        ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device="cuda") if plan["workspace_bytes"] else None
        nout = N // 2 if epi == "silu_gate" else N
        Y = torch.empty((M, nout), dtype=torch.bfloat16, device="cuda")

        def step(_, ev):
            if ev is not None:
                ev[0].record()
            qdt.quantize_per_token(X, inv, Xq, sx)
            if ev is not None:
                ev[1].record()
            qdt.w8a8_linear(Xq, sx, Wq, sw, b, epi, out=Y, workspace=ws, **kw)
            if ev is not None:
                ev[2].record()
        steps, warm = counts(step)
        info = {}
        ms, tq, tg = time_loop_best(step, steps, warm, clock_grid=plan["grid"], info=info)
        clk = info["clock"]["clock_mhz"]
        ops = 2.0 * M * N * K
        g = stats(tg)["mean"]
        r = {"M": M, "N": N, "K": K, "epilogue": epi, "plan": plan, "steps": steps, "warmup": warm,
             "ms_per_step": round(ms, 4),
             "eff_tops": round(ops / (ms * 1e-3) / 1e12, 1), "gemm_ms": round(g, 4),
             "gemm_tops": round(ops / (g * 1e-3) / 1e12, 1),
             "gemm_frac_int8_peak": round(ops / (g * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
             "gemm_clock_mhz": round(clk, 1),
             "gemm_frac_at_measured_clock": round(ops / (g * 1e-3) / 1e12 / (PEAK_INT8_TOPS * clk / 2400.0), 4),
             "quantize_ms": round(stats(tq)["mean"], 4)}
        if extra:
            r.update(extra(Y))
        res[name] = r
        log(f"{name}: {r['ms_per_step']} ms/step, GEMM {r['gemm_tops']} TOPS")

    want = (lambda n: True) if only is None else (lambda n: n == only)
    if want("dit_ffn_gate_up_4608x24576x4608"):
        d, X, Wq, sw, inv = prep("dit_ffn_gate_up_4608x24576x4608")
        Wd = to_dev(d["W_down"])

    def down(H):
        Z = torch.empty((H.shape[0], Wd.shape[0]), dtype=torch.bfloat16, device="cuda")

        def step(_, ev):
            if ev is not None:
                ev[0].record()
                ev[1].record()
            qdt.bf16_linear(H, Wd, out=Z)
            if ev is not None:
                ev[2].record()
        steps, warm = counts(step)
        _, _, tg = time_loop_best(step, steps, warm)
        g = stats(tg)["mean"]
        fl = 2.0 * H.shape[0] * Wd.shape[0] * H.shape[1]
        return {"bf16_down_proj": {"M": H.shape[0], "N": Wd.shape[0], "K": H.shape[1], "ms": round(g, 4),
                                   "tflops": round(fl / (g * 1e-3) / 1e12, 1),
                                   "frac_bf16_peak": round(fl / (g * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}}
    if want("dit_ffn_gate_up_4608x24576x4608"):
        run("dit_ffn_gate_up_4608x24576x4608", d, X, Wq, sw, inv, "silu_gate", extra=down)
        del d, X, Wq, Wd
    if want("text_cond_proj_512x4608x53248") or want("text_cond_proj_padded_4608x4608x53248"):
        d, X, Wq, sw, inv = prep("text_cond_proj_512x4608x53248")
        if want("text_cond_proj_512x4608x53248"):
            run("text_cond_proj_512x4608x53248", d, X, Wq, sw, inv, "bias")
        if want("text_cond_proj_padded_4608x4608x53248"):
            dp = W.make_workload("text_cond_proj_512x4608x53248", padded=True)
            run("text_cond_proj_padded_4608x4608x53248", dp, to_dev(dp["X"]), Wq, sw, inv, "bias")
            del dp
        del d, X, Wq
    for name in ("qk_proj_headnorm_16896x4608x4608", "qk_proj_headnorm_6037x4608x4608"):
        if want(name):
            d, X, Wq, sw, inv = prep(name)
            run(name, d, X, Wq, sw, inv, "head_rmsnorm", gamma=to_dev(d["gamma"]), eps=d["eps"])
            del d, X, Wq
    for M in (4608, 16896):
        name = f"adaln_quantize_{M}x4608"
        if want(name):
            res[name] = adaln_producer(M, 4608, counts)
    for name, src, epi in (("mxfp4_attn_proj_4608x4608x4608", "dit_attn_proj_4608x4608x4608", "bias"),
                           ("mxfp4_ffn_gate_up_4608x24576x4608", "dit_ffn_gate_up_4608x24576x4608", "silu_gate"),
                           ("mxfp4_qk_proj_headnorm_16896x4608x4608", "qk_proj_headnorm_16896x4608x4608",
                            "head_rmsnorm"),
                           ("mxfp4_text_cond_proj_512x4608x53248", "text_cond_proj_512x4608x53248", "bias")):
        if want(name):
            res[name] = mxfp4_workload(src, epi, counts)
    for bits in (4, 8):
        name = f"wo{bits}_text_cond_proj_512x4608x53248"
        if want(name):
            res[name] = weight_only_workload(bits, counts)
    for S in (4608, 16896):
        name = f"attention_{S}x18x256"
        if want(name):
            res[name] = attention_workload(S, 18, counts)
    torch.cuda.empty_cache()
    return res


def attention_workload(S, H, counts):
    """Softmax attention after the QK-norm projection over the joint sequence of S tokens, H heads
    of 256: per step one qdt_attention (V transpose pass, attention, exact-max check)."""
    import torch

    import qdt_workloads as W
    import quantized_diffusion_transformer_amd as qdt
    d = W.make_attention(S, H)
    Q, K, V = to_dev(d["Q"]), to_dev(d["K"]), to_dev(d["V"])
    ws = torch.empty(qdt.attention_workspace_size(S, H), dtype=torch.uint8, device="cuda")
    O = torch.empty((S, 256 * H), dtype=torch.bfloat16, device="cuda")

    def step(_, ev):
        if ev is not None:
            ev[0].record()
        qdt.attention(Q, K, V, H, out=O, workspace=ws)
        if ev is not None:
            ev[1].record()
            ev[2].record()
    steps, warm = counts(step)
    ms, tl, _ = time_loop_best(step, steps, warm)
    flops = 4.0 * S * S * 256 * H
    return {"S": S, "H": H, "head_dim": 256, "steps": steps, "warmup": warm, "ms_per_step": round(ms, 4),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def weight_only_workload(bits, counts):
    """The deep-K text projection with weight-only 4- or 8-bit weights (bf16 activations, half
    scales per block of 32): per step one qdt_wo_linear (GEMM over 7 fixed K slices, then the
    slice sum + bias).  Also timed: the same rows repeated to 4608, the padded call the reference
    needed for bit-exact outputs (here the 512-row call already gives the same bits)."""
    import torch

    import qdt_workloads as W
    import quantized_diffusion_transformer_amd as qdt
    d = W.make_workload("text_cond_proj_512x4608x53248")
    M, N, K = d["M"], d["N"], d["K"]
    X = to_dev(d["X"])
    Wq, Wd = qdt.wo_quantize(to_dev(d["W"]), bits)
    b = to_dev(d["bias"])

    def make_step(Xs):
        plan = qdt.wo_linear_plan(Xs.shape[0], N, K)
        ws = torch.empty(max(plan["workspace_bytes"], 16), dtype=torch.uint8, device="cuda")
        Y = torch.empty((Xs.shape[0], N), dtype=torch.bfloat16, device="cuda")

        def step(_, ev):
            if ev is not None:
                ev[0].record()
            qdt.wo_linear(Xs, Wq, Wd, b, out=Y, workspace=ws)
            if ev is not None:
                ev[1].record()
                ev[2].record()
        return step, plan
    step, plan = make_step(X)
    steps, warm = counts(step)
    ms, tl, _ = time_loop_best(step, steps, warm)
    Xp = X.repeat(9, 1)
    step_p, _ = make_step(Xp)
    steps_p, warm_p = counts(step_p)
    ms_p, _, _ = time_loop_best(step_p, steps_p, warm_p)
    ops = 2.0 * M * N * K
    wbytes = N * K * bits // 8 + N * (K // 32) * 2
    lin = stats(tl)["mean"]
    return {"M": M, "N": N, "K": K, "format": f"weight-only {bits}-bit, half scale per 32 ({bits + 0.5} bits/weight)",
            "split_k": plan["split_k"], "steps": steps, "warmup": warm, "ms_per_step": round(ms, 4),
            "linear_ms": round(lin, 4), "tflops": round(ops / (lin * 1e-3) / 1e12, 1),
            "frac_bf16_peak": round(ops / (lin * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "weight_gbs": round(wbytes / (lin * 1e-3) / 1e9, 1),
            "padded_4608_rows_ms": round(ms_p, 4), "padded_over_512_rows": round(ms_p / ms, 2)}


def mxfp4_workload(src, epi, counts):
    """Block-scaled FP4 on a workload's shapes and inputs: per step the activations are quantized
    (qdt_mxfp4_quantize) and multiplied (qdt_mxfp4_linear with epilogue `epi`); weights offline."""
    import torch

    import qdt_workloads as W
    import quantized_diffusion_transformer_amd as qdt
    d = W.make_workload(src)
    M, N, K = d["M"], d["N"], d["K"]
    X = to_dev(d["X"])
    Wq, Ws = qdt.mxfp4_quantize(to_dev(d["W"]))
    b = None if d.get("bias") is None else to_dev(d["bias"])
    Xq = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    Xs = torch.empty((K // 256, M, 8), dtype=torch.uint8, device="cuda")
    Y = torch.empty((M, N // 2 if epi == "silu_gate" else N), dtype=torch.bfloat16, device="cuda")
    g = to_dev(d["gamma"]) if epi == "head_rmsnorm" else None
    plan = qdt.mxfp4_linear_plan(M, N, K, epi)
    ws = torch.empty(max(plan["workspace_bytes"], 16), dtype=torch.uint8, device="cuda")

    def step(_, ev):
        if ev is not None:
            ev[0].record()
        qdt.mxfp4_quantize(X, None, Xq, Xs)
        if ev is not None:
            ev[1].record()
        qdt.mxfp4_linear(Xq, Xs, Wq, Ws, b, epi, gamma=g, eps=d.get("eps", 1e-6), out=Y, workspace=ws)
        if ev is not None:
            ev[2].record()
    steps, warm = counts(step)
    info = {}
    ms, tq, tg = time_loop_best(step, steps, warm, clock_grid=plan["grid"], info=info)
    clk = info["clock"]["clock_mhz"]
    ops = 2.0 * M * N * K
    g = stats(tg)["mean"]
    qb = 2 * M * K + M * K // 2 + M * K // 32
    return {"M": M, "N": N, "K": K, "format": "MXFP4 (32-element blocks, E8M0 scales)", "epilogue": epi,
            "split_k": plan["split_k"], "steps": steps, "warmup": warm, "ms_per_step": round(ms, 4),
            "eff_tops": round(ops / (ms * 1e-3) / 1e12, 1), "gemm_ms": round(g, 4),
            "gemm_tops": round(ops / (g * 1e-3) / 1e12, 1),
            "gemm_frac_fp4_peak": round(ops / (g * 1e-3) / 1e12 / PEAK_FP4_TOPS, 4),
            "gemm_clock_mhz": round(clk, 1),
            "gemm_frac_at_measured_clock": round(ops / (g * 1e-3) / 1e12 / (PEAK_FP4_TOPS * clk / 2400.0), 4),
            "quantize_ms": round(stats(tq)["mean"], 4),
            "quantize_gbs": round(qb / (stats(tq)["mean"] * 1e-3) / 1e9, 1)}


def adaln_producer(M, K, counts):
    """The producer-fused quantizer (adaLN + per-token INT8 in one pass) against the same work
    unfused (the adaLN writing bf16 h, then the quantizer reading it), on 6 rotating X buffers."""
    import torch

    import qdt_workloads as W
    import quantized_diffusion_transformer_amd as qdt
    d = W.make_adaln(M, K)
    X0 = to_dev(d["X"])
    shift, scale = to_dev(d["shift"]), to_dev(d["scale"])
    H = qdt.adaln_modulate(X0, shift, scale)
    Wq, sw, inv, _ = qdt.smooth_prepare(to_dev(d["W"]), qdt.channel_absmax(H))
    Xs = [X0] + [X0.clone() for _ in range(5)]
    Xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    it = [0]

    def fused(_, ev):
        it[0] += 1
        if ev is not None:
            ev[0].record()
        qdt.adaln_quantize(Xs[it[0] % 6], shift, scale, inv, Xq=Xq, x_scale=sx)
        if ev is not None:
            ev[1].record()
            ev[2].record()

    def unfused(_, ev):
        it[0] += 1
        if ev is not None:
            ev[0].record()
        qdt.adaln_modulate(Xs[it[0] % 6], shift, scale, H=H)
        if ev is not None:
            ev[1].record()
        qdt.quantize_per_token(H, inv, Xq, sx)
        if ev is not None:
            ev[2].record()
    steps, warm = counts(fused)
    tf, _, _ = time_loop_best(fused, steps, warm)
    tu, t_ln, t_q = time_loop_best(unfused, steps, warm)
    b = 3 * M * K + 4 * M + 4 * K + 4 * K
    return {"M": M, "K": K, "steps": steps, "warmup": warm, "fused_ms": round(tf, 4),
            "fused_gbs": round(b / (tf * 1e-3) / 1e9, 1), "fused_frac_hbm": round(b / (tf * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "unfused_ms": round(tu, 4), "unfused_adaln_ms": round(stats(t_ln)["mean"], 4),
            "unfused_quantize_ms": round(stats(t_q)["mean"], 4), "speedup": round(tu / tf, 3)}


def main():
    args = parse()
    if args.counters_from:
        summarize_counters(args.counters_from)
        return
    if args.trace_from:
        summarize_trace(args.trace_from)
        return
    if args.traffic_from:
        write_traffic(args.traffic_from)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the W8A8 linear is measured on one "
                                   "MI355X; multi-GPU sharding is a design note, not a measured path",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.only is not None and args.only != "dit_attn_proj_4608x4608x4608":
        if args.only not in EXTRA_WORKLOADS:
            print(json.dumps({"error": f"unknown workload {args.only}", "workloads": list(EXTRA_WORKLOADS)}),
                  flush=True)
            sys.exit(2)
        print(json.dumps({"workload": args.only, **extra_workloads(args, args.only)[args.only]}), flush=True)
        return
    out, d = headline(args)
    log(f"headline: {out['value']} TOPS ({out['pct_int8_peak']}% of INT8 peak), {out['ms_per_step']} ms/step")
    if args.only is None and not args.no_extra:
        try:
            out["other_workloads"] = extra_workloads(args)
        except Exception as e:  # the headline line is still reported
            out["other_workloads"] = {"error": repr(e)}
    if not args.no_cpu_baseline and args.only is None:
        log("cpu baseline (oracle on the host)")
        out["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
