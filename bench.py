"""Benchmark: fused SDPA forward TFLOP/s on MI355X (one GPU).

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu-baseline]

A step is one launch of the forward over the headline workload: causal bf16
attention at b4 h16 s1024 d64, BHSD, scale 1/8, inputs iid N(0,1) from a fixed
seed, already resident in HBM. W untimed launches, then exactly K timed steps,
each one a 512 MiB write (which evicts the L2 caches and the MALL) followed by
the launch, bracketed by device synchronisation. The device time of each
launch comes from the kernel trace that torch's profiler collects through
ROCm's tracer (the kernel's own begin and end); `value` and `ms_per_step` are
the MEDIAN over the K steps and `roofline.achieved` uses the MEAN [kernel-trace].
As a cross-check, HIP events on the launch stream time K x (flush + launch)
and K x flush alone; their difference / K is reported as
`roofline.events_mean_launch_ms` (and becomes the figure, tagged [hip-events],
if the trace is unavailable). Warm-cache figures (back-to-back launches,
caches holding the inputs) are reported separately, labelled, under `extra`.

FLOP count: the pages' formula 4*b*h*s^2*d, halved when causal ("Inside
NVIDIA's cuDNN Graph API ...", section 5). Roofline: MFMA-bound against the
dense bf16 peak of 2500 TFLOP/s.

One JSON line is printed. Besides the headline it carries:
  roofline      achieved/peak of the forward kernel, and its HBM traffic from
                the committed rocprofv3 counter summary when that summary was
                taken on the current kernel source (else null);
  cpu_baseline  the fp64 oracle timed on this host's cores: the headline
                workload (`value`), and under `per_workload` every workload
                (all host threads) plus the two forward workloads of the
                first kind single-threaded; a baseline, not the target;
  extra         warm-cache figures of the headline, and cold and warm figures
                of the other workloads (fp32 b1h2s128d64, bf16/fp16
                non-causal b2h16s4096d128 BSHD, packed causal bf16 32
                sequences h16 d128, e4m3 forward on two shapes, causal bf16
                backward b4h16s2048d128).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0  # dense e4m3 MFMA peak of MI355X
PEAK_HBM_GBS = 8000.0
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "fwd_bf16_b4h16s1024d64_causal_counters.json")
FWD_SOURCES = [os.path.join(ROOT, "scaled_dot_product_07_amd", "csrc", f)
               for f in ("fwd.hip", "fwd_common.h", "kernel_common.h")]


COPY_BYTES = 256 << 20  # calibration copy: reads and writes this many bytes
FWD_KERNEL_TAG = "fwd16_kernel"


def _pmc_means(root, counter):
    """Mean counter value per dispatch for the forward kernel and for the copy kernel."""
    import csv
    import glob
    fwd, cp = [], []
    for f in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] != counter:
                continue
            name, val = row["Kernel_Name"], float(row["Counter_Value"])
            if FWD_KERNEL_TAG in name and "DF16b" in name and "Li64ELb1ELb0" in name:
                fwd.append(val)
            elif "copy" in name.lower() and "fill" not in name.lower():
                cp.append(val)
    if not fwd or not cp:
        raise SystemExit(f"{root}: {counter} rows missing (fwd {len(fwd)}, copy {len(cp)})")
    return sum(fwd) / len(fwd), sum(cp) / len(cp), len(fwd)


def summarize_counters(fetch_dir, write_dir):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the headline forward, each
    scaled by bytes / counter of a plain copy of COPY_BYTES, written next to the
    forward's source digest (a summary taken on other source is not used)."""
    f_fwd, f_cp, n_f = _pmc_means(fetch_dir, "FETCH_SIZE")
    w_fwd, w_cp, n_w = _pmc_means(write_dir, "WRITE_SIZE")
    kf = COPY_BYTES / (f_cp * 1024.0)
    kw = COPY_BYTES / (w_cp * 1024.0)
    read_b = f_fwd * 1024.0 * kf
    write_b = w_fwd * 1024.0 * kw
    out = {
        "kernel": "fwd16_kernel<bf16, d64, causal, dense>",
        "workload": "b4 h16 s1024 d64 causal bf16 BHSD",
        "fwd_source_sha256_16": source_digest(FWD_SOURCES),
        "fetch_kib_per_dispatch": f_fwd, "write_kib_per_dispatch": w_fwd,
        "copy_fetch_kib": f_cp, "copy_write_kib": w_cp, "copy_bytes": COPY_BYTES,
        "fetch_scale": kf, "write_scale": kw,
        "hbm_read_bytes_per_launch": read_b, "hbm_write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": read_b + write_b,
        "algorithmic_bytes_per_launch": 4 * 4 * 16 * 1024 * 64 * 2 + 4 * 16 * 1024 * 4,
        "dispatches": [n_f, n_w],
    }
    os.makedirs(os.path.dirname(TRAFFIC_SUMMARY), exist_ok=True)
    with open(TRAFFIC_SUMMARY, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def fwd_flops(b, h, s_q, s_kv, d, causal):
    f = 4.0 * b * h * s_q * s_kv * d
    return f * 0.5 if causal else f


def source_digest(paths):
    """First 16 hex digits of the SHA-256 of the forward kernel's sources."""
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def time_launches(fn, steps, warmup, torch, graph=True):
    """Mean ms per call over `steps` back-to-back calls, HIP events on the launch stream.

    graph=True captures the `steps` calls into one HIP graph and times one
    replay, so host-side launch cost (Python, ctypes) cannot starve the GPU;
    graph=False times the calls issued eagerly from Python.
    """
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                fn()
        g.replay()  # untimed: first replay uploads the graph
        torch.cuda.synchronize()
        start.record()
        g.replay()
        stop.record()
    else:
        start.record()
        for _ in range(steps):
            fn()
        stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def _is_ours(name: str) -> bool:
    """Kernels of this library (all live in namespace sdpa07)."""
    return "sdpa07" in name


def time_cold(fn, iters, torch, flush, trace=True):
    """Cold-cache timing of `iters` calls, each preceded by writing the whole
    `flush` buffer (512 MiB: evicts the L2 caches and the MALL).

    Two measurements of the same kind of timed region:
      trace   per-call device time of this library's kernels (summed over the
              kernels of one call) from the kernel trace that torch's profiler
              collects through ROCm's tracer: median and mean;
      events  HIP events on the launch stream around `iters` x (flush + call)
              and around `iters` x flush alone; their difference / iters is
              the mean device time per call (launches queue back to back, so no
              dispatch gap is counted; events around one launch would include
              the launch latency).
    Returns a dict of ms figures; the trace part is None when the profiler
    yields no kernel records."""
    out = {"trace_median_ms": None, "trace_mean_ms": None}
    torch.cuda.synchronize()
    try:
        if not trace:
            raise RuntimeError("kernel trace switched off (--no-trace)")
        from torch.profiler import ProfilerActivity, profile
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            for i in range(iters):
                flush.fill_(i & 0x7f)
                fn()
            torch.cuda.synchronize()
        per_call, cur, seen = [], 0.0, False
        for e in sorted((e for e in prof.events() if e.device_type.name == "CUDA"),
                        key=lambda e: e.time_range.start):
            if _is_ours(e.name):
                cur += (e.time_range.end - e.time_range.start) * 1e-3
                seen = True
            elif seen:
                per_call.append(cur)
                cur, seen = 0.0, False
        if seen:
            per_call.append(cur)
        if len(per_call) == iters:
            out["trace_median_ms"] = float(np.median(per_call))
            out["trace_mean_ms"] = float(np.mean(per_call))
    except Exception as ex:  # reported, never hidden
        out["trace_error"] = repr(ex)[:200]

    def region(with_call):
        a = torch.cuda.Event(enable_timing=True)
        z = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(iters):
            flush.fill_(i & 0x7f)
            if with_call:
                fn()
        z.record()
        torch.cuda.synchronize()
        return a.elapsed_time(z)

    t_both, t_flush = region(True), region(False)
    out["events_mean_ms"] = (t_both - t_flush) / iters
    return out


def traffic_from_counters():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when it is missing or was taken on a different forward kernel source."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return None
    if s.get("fwd_source_sha256_16") != source_digest(FWD_SOURCES):
        return None
    return s.get("hbm_bytes_per_launch")


def _oracle_rate(fn, flops, min_seconds, max_reps):
    """(TFLOP/s, repetitions, seconds) of fn() repeated until min_seconds pass."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= max_reps:
            return flops * reps / el / 1e12, reps, el


def cpu_baseline(W, quick=False):
    """The fp64 oracle on the same inputs as the GPU workloads, on this host.

    Every workload runs on all host threads (the headline one repeated for about
    2 s, the larger ones once); the fp32 and the headline workloads also run on
    one thread. Inputs are the fp64 upcast of the very bytes the GPU gets."""
    import torch
    import oracle
    threads = oracle.hardware_threads()
    f64 = lambda t: t.to(torch.float64).contiguous().numpy()  # noqa: E731
    per = {}

    def dense(case, nthreads, min_s, max_reps):
        q, k, v = (f64(x) for x in W.case_inputs(case))
        flops = fwd_flops(case.b, case.h, case.s_q, case.s_kv, case.d, case.causal)
        tf, reps, el = _oracle_rate(
            lambda: oracle.fwd(q, k, v, case.scale, case.causal, threads=nthreads), flops,
            min_s, max_reps)
        return {"tflops": round(tf, 6), "cores": nthreads, "repetitions": reps,
                "seconds": round(el, 3)}

    c2 = W.FWD_BF16_B4H16S1024D64
    head = dense(c2, threads, 2.0, 50)
    per["fwd_bf16_b4h16s1024d64_causal"] = head
    per["fwd_bf16_b4h16s1024d64_causal_1thread"] = dense(c2, 1, 1.0, 3)
    per["fwd_fp32_b1h2s128d64_causal"] = dense(W.FWD_FP32_B1H2S128D64, threads, 0.5, 200)
    per["fwd_fp32_b1h2s128d64_causal_1thread"] = dense(W.FWD_FP32_B1H2S128D64, 1, 0.5, 200)
    if not quick:
        per["fwd_bf16_b2h16s4096d128_bshd"] = dense(W.FWD_BF16_B2H16S4096D128, threads, 0.0, 1)
        c = W.VARLEN_BF16_32SEQ_H16D128
        inp = W.varlen_case_inputs(c, poison_tail=False)
        q, k, v = (f64(x) for x in (inp.q, inp.k, inp.v))
        lens = inp.lens_q.double()
        vflops = float((4.0 * c.h * lens * lens * c.d * 0.5).sum())
        tf, reps, el = _oracle_rate(
            lambda: oracle.fwd_varlen(q, k, v, inp.cu_q.numpy(), inp.cu_kv.numpy(), c.scale, True,
                                      threads=threads), vflops, 0.0, 1)
        per["fwd_varlen_bf16_32seq_h16d128_causal"] = {
            "tflops": round(tf, 6), "cores": threads, "repetitions": reps, "seconds": round(el, 3)}
        # the backward on a sample: batch 0, heads 0-7 (1/8 of the workload)
        c = W.BWD_BF16_B4H16S2048D128
        q, k, v, do = (f64(x[:1, :8]) for x in W.case_inputs(c))
        bflops = 2.5 * fwd_flops(1, 8, c.s_q, c.s_kv, c.d, True)
        tf, reps, el = _oracle_rate(
            lambda: oracle.bwd(q, k, v, do, c.scale, True, threads=threads), bflops, 0.0, 1)
        per["bwd_bf16_b4h16s2048d128_causal"] = {
            "tflops": round(tf, 6), "cores": threads, "repetitions": reps, "seconds": round(el, 3),
            "sample": "batch 0, heads 0-7 of the workload (1/8 of it)",
            "flop_convention": "2.5x the forward count; the oracle also recomputes its forward"}
    return {"value": head["tflops"], "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"the full b4 h16 s1024 d64 causal workload (fp64 upcast of the same bf16 "
                      f"inputs), {head['repetitions']} repetitions in {head['seconds']} s on "
                      f"{threads} threads; per_workload: every workload once at full size (the "
                      f"backward on 8 of its 64 heads)",
            "per_workload": per}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick-cpu-baseline", action="store_true",
                    help="time the oracle on the two small forward workloads only")
    ap.add_argument("--no-trace", action="store_true",
                    help="time with HIP events only (when an outside profiler traces the run)")
    ap.add_argument("--warm", action="store_true",
                    help="time back-to-back launches without the cache flush (for counters)")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="also run a plain device copy of COPY_BYTES (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script "
                         "with --copy-calibrate into the HBM traffic summary, then exit")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import scaled_dot_product_07_amd as sdpa
    import workloads as W

    dev = torch.device("cuda", 0)
    c = W.FWD_BF16_B4H16S1024D64
    q, k, v = W.case_inputs(c)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty(c.b, c.h, c.s_q, device=dev, dtype=torch.float32)

    def step():
        sdpa.fwd(qd, kd, vd, scale=c.scale, causal=c.causal, out=o, lse=lse)

    flops = fwd_flops(c.b, c.h, c.s_q, c.s_kv, c.d, c.causal)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.warm:
        ms = ms_mean = time_launches(step, args.steps, 0, torch, graph=False)
        timing = "warm: back-to-back launches, mean [hip-events]"
        cold = None
    else:
        cold = time_cold(step, args.steps, torch, flush, trace=not args.no_trace)
        if cold["trace_median_ms"] is not None:
            ms, ms_mean = cold["trace_median_ms"], cold["trace_mean_ms"]
            timing = ("cold: 512 MiB written before each launch; device time of the kernel from "
                      "the kernel trace (torch profiler over ROCm's tracer): value = median, "
                      "roofline = mean [kernel-trace]")
        else:
            ms = ms_mean = cold["events_mean_ms"]
            timing = ("cold: 512 MiB written before each launch; mean device time from HIP events "
                      "(K x (flush + launch) minus K x flush) [hip-events]")
    tflops = flops / (ms * 1e-3) / 1e12
    tflops_mean = flops / (ms_mean * 1e-3) / 1e12
    traffic = traffic_from_counters()
    result = {
        "metric": "SDPA fwd TFLOP/s, b4 h16 s1024 d64 causal bf16; % of MFMA peak",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (iid N(0,1) from seed 1002, cast to bf16)",
        "config": {"workload": "fused SDPA forward, causal, BHSD", "b": c.b, "h": c.h,
                   "s": c.s_q, "d": c.d, "scale": c.scale, "flop_per_step": flops,
                   "timing": timing},
        "roofline": {"bound": "mfma", "achieved": round(tflops_mean, 3),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops_mean / PEAK_BF16_TFLOPS, 4),
                     "mean_launch_ms": round(ms_mean, 6), "traffic": traffic},
    }
    if cold is not None:
        result["roofline"]["events_mean_launch_ms"] = round(cold["events_mean_ms"], 6)
        if "trace_error" in cold:
            result["roofline"]["trace_error"] = cold["trace_error"]

    extra = {}
    if not args.no_extra:
        w_graph = time_launches(step, 500, 20, torch, graph=True)
        w_eager = time_launches(step, 500, 20, torch, graph=False)
        extra["fwd_bf16_b4h16s1024d64_causal_warm"] = {
            "label": "warm cache (no flush), back-to-back launches [hip-events]",
            "graph_replay_ms": round(w_graph, 6), "eager_ms": round(w_eager, 6),
            "tflops_graph_replay": round(flops / (w_graph * 1e-3) / 1e12, 3)}
        extra.update(bench_other_workloads(torch, sdpa, W, dev, flush, not args.no_trace))
    del flush
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(W, quick=args.quick_cpu_baseline)
    if extra:
        result["extra"] = extra
    if args.copy_calibrate:
        src = torch.ones(COPY_BYTES // 4, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps(result), flush=True)


def _both(fn, flops, torch, flush, cold_iters=20, warm_iters=50, trace=True):
    """Cold (flushed; kernel-trace median, else HIP-event mean) and warm
    (back-to-back graph replay, HIP-event mean) figures."""
    for _ in range(3):
        fn()
    c = time_cold(fn, cold_iters, torch, flush, trace=trace)
    cold = c["trace_median_ms"] if c["trace_median_ms"] is not None else c["events_mean_ms"]
    warm = time_launches(fn, warm_iters, 3, torch, graph=True)
    tc = flops / (cold * 1e-3) / 1e12
    tw = flops / (warm * 1e-3) / 1e12
    return {"cold_ms": round(cold, 6), "tflops": round(tc, 3),
            "frac_of_mfma_peak": round(tc / PEAK_BF16_TFLOPS, 4),
            "cold_events_mean_ms": round(c["events_mean_ms"], 6),
            "warm_ms": round(warm, 6), "warm_tflops": round(tw, 3)}


def bench_other_workloads(torch, sdpa, W, dev, flush, trace=True):
    out = {}
    both = lambda *a, **kw: _both(*a, trace=trace, **kw)  # noqa: E731
    # fp32 causal b1 h2 s128 d64 (latency-bound correctness workload)
    c = W.FWD_FP32_B1H2S128D64
    q, k, v = (x.to(dev) for x in W.case_inputs(c))
    out["fwd_fp32_b1h2s128d64_causal"] = both(
        lambda: sdpa.fwd(q, k, v, scale=c.scale, causal=True), fwd_flops(1, 2, 128, 128, 64, True),
        torch, flush)
    # non-causal b2 h16 s4096 d128 BSHD, bf16 and fp16
    for c in (W.FWD_BF16_B2H16S4096D128, W.FWD_FP16_B2H16S4096D128):
        q, k, v = (x.to(dev) for x in W.case_inputs(c))
        o = torch.empty_like(q)
        out[f"fwd_{c.dtype}_b2h16s4096d128_bshd"] = both(
            lambda: sdpa.fwd(q, k, v, scale=c.scale, causal=False, out=o),
            fwd_flops(c.b, c.h, c.s_q, c.s_kv, c.d, False), torch, flush)
        del q, k, v, o
    # packed causal bf16, 32 sequences
    c = W.VARLEN_BF16_32SEQ_H16D128
    inp = W.varlen_case_inputs(c)
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    cu = inp.cu_q.to(dev)
    mx = int(inp.lens_q.max())
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[0], c.h, device=dev, dtype=torch.float32)
    lens = inp.lens_q.double()
    vflops = float((4.0 * c.h * lens * lens * c.d * 0.5).sum())
    e = both(lambda: sdpa.fwd_varlen(q, k, v, cu, cu, mx, mx, total_q=inp.total_q,
                                      total_kv=inp.total_kv, scale=c.scale, causal=True, out=o,
                                      lse=lse), vflops, torch, flush)
    e["total_tokens"] = inp.total_q
    out["fwd_varlen_bf16_32seq_h16d128_causal"] = e
    del q, k, v, o, lse
    # the two dense forward shapes with e4m3 inputs (the workloads' values
    # rounded to e4m3), bf16 output; priced against the fp8 MFMA peak
    for c, layout in ((W.FWD_BF16_B4H16S1024D64, "causal"), (W.FWD_BF16_B2H16S4096D128, "bshd")):
        q, k, v = (x.to(dev).to(torch.float8_e4m3fn) for x in W.case_inputs(c))
        o = torch.empty(q.shape, device=dev, dtype=torch.bfloat16)
        e = both(lambda: sdpa.fwd_fp8(q, k, v, scale=c.scale, causal=c.causal, out=o,
                                       return_lse=False),
                  fwd_flops(c.b, c.h, c.s_q, c.s_kv, c.d, c.causal), torch, flush)
        e["frac_of_fp8_mfma_peak"] = round(e["tflops"] / PEAK_FP8_TFLOPS, 4)
        out[f"fwd_fp8_b{c.b}h{c.h}s{c.s_q}d{c.d}_{layout}"] = e
        del q, k, v, o
    # causal bf16 backward b4 h16 s2048 d128 (two kernels per call)
    c = W.BWD_BF16_B4H16S2048D128
    q, k, v, do = (x.to(dev) for x in W.case_inputs(c))
    o, lse = sdpa.fwd(q, k, v, scale=c.scale, causal=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(sdpa.bwd_workspace_size(c.b, c.h, c.s_q, c.d, q.dtype),
                     dtype=torch.uint8, device=dev)
    e = both(lambda: sdpa.bwd(q, k, v, o, do, lse, scale=c.scale, causal=True, dq=dq, dk=dk,
                               dv=dv, workspace=ws),
              2.5 * fwd_flops(c.b, c.h, c.s_q, c.s_kv, c.d, True), torch, flush, cold_iters=10,
              warm_iters=20)
    e["flop_convention"] = "2.5x the forward count (five products of the backward)"
    out["bwd_bf16_b4h16s2048d128_causal"] = e
    return out


if __name__ == "__main__":
    main()
