"""Benchmark: fused SDPA forward TFLOP/s on MI355X (one GPU).

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu-baseline]

A step is one launch of the forward over the headline workload: causal bf16
attention at b4 h16 s1024 d64, BHSD, scale 1/8, inputs iid N(0,1) from a fixed
seed, already resident in HBM. W untimed steps, then exactly K steps timed with
HIP events recorded on the launch stream (torch's current stream, which the
binding launches on), bracketed by device synchronisation. The K launches are
captured into one HIP graph and replayed once inside the timed region, so the
host's per-call cost does not leave the GPU idle between launches.

FLOP count: the pages' formula 4*b*h*s^2*d, halved when causal ("Inside
NVIDIA's cuDNN Graph API ...", section 5). Roofline: MFMA-bound against the
dense bf16 peak of 2500 TFLOP/s.

One JSON line is printed. Besides the headline it carries:
  roofline      achieved/peak of the forward kernel, and its HBM traffic from
                the committed rocprofv3 counter summary when that summary was
                taken on the current kernel source (else null);
  cpu_baseline  the fp64 oracle timed on this host's cores on the same
                workload (a baseline, not the target);
  extra         the other workloads (fp32 b1h2s128d64, bf16/fp16 non-causal
                b2h16s4096d128 BSHD, packed causal bf16 32 sequences h16 d128,
                causal bf16 backward b4h16s2048d128) and a cold-cache timing of
                the headline (512 MiB written between launches).
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


def time_cold(fn, iters, torch, flush_bytes=512 << 20):
    """Median ms of single calls, each after writing `flush_bytes` (evicts L2 and MALL)."""
    buf = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    ts = []
    for _ in range(iters):
        buf.fill_(1)
        a = torch.cuda.Event(enable_timing=True)
        z = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        z.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(z))
    del buf
    return float(np.median(ts))


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


def cpu_baseline(q, k, v, scale, causal, flops_full, min_seconds=10.0):
    """The fp64 oracle on the same workload, repeated until min_seconds elapse."""
    import torch
    import oracle
    q64, k64, v64 = (x.to(torch.float64).contiguous().numpy() for x in (q, k, v))
    threads = oracle.hardware_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.fwd(q64, k64, v64, scale, causal, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= 50:
            break
    return {"value": round(flops_full * reps / el / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads, "kind": "oracle",
            "sample": f"the full b4 h16 s1024 d64 causal workload (fp64 upcast of the same bf16 "
                      f"inputs), {reps} repetitions in {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of one graph replay (for profilers)")
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

    ms = time_launches(step, args.steps, args.warmup, torch, graph=not args.no_graph)
    flops = fwd_flops(c.b, c.h, c.s_q, c.s_kv, c.d, c.causal)
    tflops = flops / (ms * 1e-3) / 1e12
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
                   "s": c.s_q, "d": c.d, "scale": c.scale, "flop_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }

    extra = {}
    if not args.no_extra:
        extra["fwd_bf16_b4h16s1024d64_causal_eager_ms"] = round(
            time_launches(step, args.steps, 10, torch, graph=False), 6)
        extra["fwd_bf16_b4h16s1024d64_causal_cold_ms"] = round(time_cold(step, 50, torch), 6)
        extra.update(bench_other_workloads(torch, sdpa, W, dev))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(q, k, v, c.scale, c.causal, flops)
    if extra:
        result["extra"] = extra
    if args.copy_calibrate:
        src = torch.ones(COPY_BYTES // 4, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps(result), flush=True)


def bench_other_workloads(torch, sdpa, W, dev):
    out = {}
    # fp32 causal b1 h2 s128 d64 (latency-bound correctness workload)
    c = W.FWD_FP32_B1H2S128D64
    q, k, v = (x.to(dev) for x in W.case_inputs(c))
    ms = time_launches(lambda: sdpa.fwd(q, k, v, scale=c.scale, causal=True), 200, 20, torch)
    out["fwd_fp32_b1h2s128d64_causal"] = _entry(ms, fwd_flops(1, 2, 128, 128, 64, True))
    # non-causal b2 h16 s4096 d128 BSHD, bf16 and fp16
    for c in (W.FWD_BF16_B2H16S4096D128, W.FWD_FP16_B2H16S4096D128):
        q, k, v = (x.to(dev) for x in W.case_inputs(c))
        o = torch.empty_like(q)
        ms = time_launches(lambda: sdpa.fwd(q, k, v, scale=c.scale, causal=False, out=o),
                           50, 5, torch)
        out[f"fwd_{c.dtype}_b2h16s4096d128_bshd"] = _entry(
            ms, fwd_flops(c.b, c.h, c.s_q, c.s_kv, c.d, False))
        del q, k, v, o
    # packed causal bf16, 32 sequences
    c = W.VARLEN_BF16_32SEQ_H16D128
    inp = W.varlen_case_inputs(c)
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    cu = inp.cu_q.to(dev)
    mx = int(inp.lens_q.max())
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[0], c.h, device=dev, dtype=torch.float32)
    ms = time_launches(lambda: sdpa.fwd_varlen(q, k, v, cu, cu, mx, mx, total_q=inp.total_q,
                                               total_kv=inp.total_kv, scale=c.scale,
                                               causal=True, out=o, lse=lse), 50, 5, torch)
    lens = inp.lens_q.double()
    vflops = float((4.0 * c.h * lens * lens * c.d * 0.5).sum())
    e = _entry(ms, vflops)
    e["total_tokens"] = inp.total_q
    out["fwd_varlen_bf16_32seq_h16d128_causal"] = e
    # the two dense forward shapes with e4m3 inputs (the workloads' values
    # rounded to e4m3), bf16 output; priced against the fp8 MFMA peak
    for c, layout in ((W.FWD_BF16_B4H16S1024D64, "causal"), (W.FWD_BF16_B2H16S4096D128, "bshd")):
        q, k, v = (x.to(dev).to(torch.float8_e4m3fn) for x in W.case_inputs(c))
        o = torch.empty(q.shape, device=dev, dtype=torch.bfloat16)
        ms = time_launches(lambda: sdpa.fwd_fp8(q, k, v, scale=c.scale, causal=c.causal, out=o,
                                                return_lse=False), 50, 5, torch)
        e = _entry(ms, fwd_flops(c.b, c.h, c.s_q, c.s_kv, c.d, c.causal))
        e["frac_of_fp8_mfma_peak"] = round(e["tflops"] / PEAK_FP8_TFLOPS, 4)
        out[f"fwd_fp8_b{c.b}h{c.h}s{c.s_q}d{c.d}_{layout}"] = e
        del q, k, v, o
    # causal bf16 backward b4 h16 s2048 d128
    c = W.BWD_BF16_B4H16S2048D128
    q, k, v, do = (x.to(dev) for x in W.case_inputs(c))
    try:
        o, lse = sdpa.fwd(q, k, v, scale=c.scale, causal=True)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(sdpa.bwd_workspace_size(c.b, c.h, c.s_q, c.d, q.dtype),
                         dtype=torch.uint8, device=dev)
        ms = time_launches(lambda: sdpa.bwd(q, k, v, o, do, lse, scale=c.scale, causal=True,
                                            dq=dq, dk=dk, dv=dv, workspace=ws), 20, 3, torch)
        e = _entry(ms, 2.5 * fwd_flops(c.b, c.h, c.s_q, c.s_kv, c.d, True))
        e["flop_convention"] = "2.5x the forward count (five products of the backward)"
        out["bwd_bf16_b4h16s2048d128_causal"] = e
    except Exception as ex:  # reported, never hidden
        out["bwd_bf16_b4h16s2048d128_causal"] = {"error": str(ex)}
    return out


def _entry(ms, flops):
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 6), "tflops": round(tf, 3),
            "frac_of_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


if __name__ == "__main__":
    main()
