#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

A step is one fused streaming forward (attn_fwd) over the whole workload:
batch 1 x 32 heads, N = 16384, d = 128, bf16 inputs drawn iid N(0, 1) with Q
multiplied by 4 (large score ranges), fp32 accumulation, scale 1/sqrt(d).
Inputs are resident in HBM before timing starts.  W warmup steps run
untimed; then K steps are timed back to back between two device
synchronisations, and each launch is also bracketed by HIP events on the
stream the kernel runs on.

Reported (one JSON line on stdout):
  value        whole-job TFLOP/s, 4 N^2 d flops per head (both products, mul
               and add counted apart) / mean step time;
  roofline     the fused kernel against the dense bf16 MFMA peak (2.5
               PFLOP/s): achieved = algorithmic flops per launch / mean launch
               time from the HIP events; traffic = HBM bytes per launch from
               the committed rocprofv3 counter summary when it was taken on
               the current kernel source, else null;
  hbm_gbps     compulsory bytes (Q, K, V read once, O and lse written once) /
               step time, and as a fraction of 8 TB/s; l2miss_gbps the
               measured L2-miss bytes (traffic) / launch time;
  launch_ms_*  min, median, p90, max over the timed launches, and
               cold_launch_ms with L2 and MALL flushed by a 512 MB write;
  measured_peaks  a library bf16 GEMM, a device copy, the library's
               matrix-core loop (random and zero operands) and its
               streaming read (2 GiB) on the same GPU, the reachable rates
               beside the published peaks (the decoding leg also reports
               its bandwidth as a fraction of the streaming read);
  cpu_baseline the float64 oracle on the host cores, on a bounded sample of
               rows of the same workload (about 15 s of CPU work);
  secondary    the small-cache square-tile path (batch 1 x 8 heads, N 4096,
               d 256), the backward (batch 2 x 16 heads, N 4096, d 128) and
               the other paths, when built (not part of `value`): each leg
               warmed up for 0.3 s, then K back-to-back calls between one
               pair of HIP events (per-call event pairs would add about
               10 us of device time to each sub-millisecond call).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-secondary]
                       [--legs a,b] [--secondary-only]
       python bench.py --calibrate-copy          (copy kernel for counter scaling)
       python bench.py --profile-leg LEG [--calls C]  (one leg, for a counter run)
       python bench.py --summarize-leg-counters DIR  (write the per-leg traffic summary)
       python bench.py --tile-sweep [--steps K]   (fused forward at B_r x B_c shapes)
       python bench.py --summarize-sweep DIR TIMING.jsonl OUT.md  (sweep table)
       python bench.py --smallcache-sweep [--steps K]   (square tiles at each b, d = 256)
       python bench.py --summarize-smallcache-sweep DIR TIMING.jsonl OUT.md
       python bench.py --bwd-tile-sweep [--steps K]   (blockwise backward at each tile shape)
       python bench.py --summarize-bwd-sweep DIR TIMING.jsonl OUT.md
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published
HEADLINE = "fwd_bf16_b1h32_n16384_d128_qx4"
METRIC = "attention fwd TFLOP/s (4N²d/head) and % of bf16 MFMA peak; HBM GB/s at 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
COPY_BYTES = 1 << 30  # counter calibration: bytes read and written per copy
SECONDARY_WARM_S = 0.3  # warm-up of each secondary leg before it is timed
COMMON_SOURCES = ["aware_tiling_amd/csrc/device_common.h", "aware_tiling_amd/csrc/index_maps.h",
                  "aware_tiling_amd/csrc/lds_dma.h"]
# Per leg: the kernel sources its counter bytes are keyed by, and the kernel
# name substrings that make up one call (the forward calls that produce a
# backward leg's O and lse are not among them).
LEGS = {
    "headline": (["aware_tiling_amd/csrc/fwd_fused.hip"], ("fwd_fused_bf16",)),
    "smallcache": (["aware_tiling_amd/csrc/fwd_smallcache.hip"],
                   ("sc_scores_exp", "sc_value_product")),
    "backward": (["aware_tiling_amd/csrc/bwd.hip"], ("bwd_preprocess", "bwd_dkdv3", "bwd_dq3")),
    "backward_d256": (["aware_tiling_amd/csrc/bwd.hip"],
                      ("bwd_preprocess", "bwd_dkdv3", "bwd_dq3")),
    "smallcache_backward_d256": (["aware_tiling_amd/csrc/bwd_smallcache.hip",
                                  "aware_tiling_amd/csrc/bwd.hip"], ("bwd_preprocess", "sb_")),
    "smallcache_backward_d128": (["aware_tiling_amd/csrc/bwd_smallcache.hip",
                                  "aware_tiling_amd/csrc/bwd.hip"], ("bwd_preprocess", "sb_")),
}
SMALLCACHE_M = 49152  # 3/4 of d^2 at d = 256: the small-cache regime M < d^2
SMALLCACHE_BWD = {"smallcache_backward_d256": ("bwd_smallcache_bf16_b1h8_n4096_d256", 49152),
                  "smallcache_backward_d128": ("bwd_bf16_b2h16_n4096_d128", 12288)}
# the blockwise (large-cache) backward on its own workload and on the d = 256
# workload of the small-cache backward
BLOCKWISE_BWD = {"backward": "bwd_bf16_b2h16_n4096_d128",
                 "backward_d256": "bwd_smallcache_bf16_b1h8_n4096_d256"}


def kernel_digest(leg: str = "headline") -> str:
    """Digest of the sources a leg's kernels are built from."""
    h = hashlib.sha256()
    for p in COMMON_SOURCES + LEGS[leg][0]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def time_launches(fn, steps: int, warmup: int, batch: bool = False, warm_s: float = 0.0):
    """Mean ms per launch from HIP events on the current stream, and the
    wall-clock ms per step between synchronisations.

    Default: every launch bracketed by its own pair of events (the per-launch
    distribution).  batch=True: one pair of events around the `steps`
    back-to-back launches, for sub-millisecond paths, where an event pair
    between launches costs about 10 us of device time.  warm_s: keep warming
    up for that many seconds after the `warmup` launches (the clocks of an
    idle GPU ramp up over the first tens of milliseconds of work)."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if warm_s > 0:
        t_end = time.perf_counter() + warm_s
        while time.perf_counter() < t_end:
            for _ in range(8):
                fn()
            torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    if batch:
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        s.record(stream)
        for _ in range(steps):
            fn()
        e.record(stream)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
        ms = s.elapsed_time(e) / steps
        return ms, wall_ms, [ms]
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ev = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return sum(ev) / len(ev), wall_ms, ev


def percentile(xs, p):
    ys = sorted(xs)
    i = min(len(ys) - 1, max(0, int(round(p / 100.0 * (len(ys) - 1)))))
    return ys[i]


def cold_launch_ms(fn, torch, dev, reps: int = 5) -> float:
    """Median launch time with the caches flushed first: a 512 MB buffer is
    written before each launch (more than L2 and the 256 MB MALL), and the
    HIP events bracket the launch alone."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        flush.fill_(1)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        fn()
        e.record(stream)
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    del flush
    return percentile(times, 50)


def measured_peaks(torch, dev, at=None) -> dict:
    """Reference rates measured on this device: a library bf16 GEMM
    (8192^3, torch.matmul), a 1 GiB device-to-device copy and, when the
    library is built, its matrix-core loop (the attention kernels' MFMA
    instruction on register operands, no memory traffic) with random bf16
    operands and with zero operands, at two waves per SIMD, and its
    streaming read of 2 GiB (best of three grid sizes)."""
    loops = {}
    if at is not None:
        out = torch.empty(512 * 256, dtype=torch.float32, device=dev)
        for name, amp in (("mfma_loop_bf16_tflops", 1.0), ("mfma_loop_zero_data_bf16_tflops", 0.0)):
            flops = [0]
            def run():
                flops[0] = at.calib_mfma_loop(out, 100000, amp)
            ms, _, _ = time_launches(run, 5, 2)
            loops[name] = round(flops[0] / (ms * 1e-3) / 1e12, 1)
        del out
    a = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
    b = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
    gemm_ms, _, _ = time_launches(lambda: torch.matmul(a, b), 10, 3)
    del a, b
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    copy_ms, _, _ = time_launches(lambda: dst.copy_(src), 10, 3)
    del src, dst
    if at is not None:
        # streaming read of 2 GiB, the best of three grid sizes
        src = torch.ones(2 * COPY_BYTES, dtype=torch.uint8, device=dev)
        best = 0.0
        for wgs in (1024, 2048, 4096):
            out = torch.empty(wgs * 256, dtype=torch.int32, device=dev)
            ms, _, _ = time_launches(lambda: at.calib_stream_read(src, out), 10, 3)
            best = max(best, 2 * COPY_BYTES / (ms * 1e-3) / 1e9)
            del out
        loops["stream_read_gbps"] = round(best, 1)
        del src
    torch.cuda.empty_cache()
    return {"gemm_bf16_tflops": round(2 * 8192 ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
            "copy_gbps": round(2 * COPY_BYTES / (copy_ms * 1e-3) / 1e9, 1), **loops}


def leg_traffic(leg: str):
    """The committed counter summary of one leg (HBM bytes per call, read and
    written), if it was taken on the leg's current kernel sources, else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get("legs", {}).get(leg)
    except (OSError, ValueError):
        return None
    if not t or t.get("kernel_digest") != kernel_digest(leg):
        return None
    return t


def traffic_for_launch():
    """HBM bytes per launch of the headline kernel (None when stale)."""
    t = leg_traffic("headline")
    return t["bytes_per_call"] if t else None


def leg_call(leg: str, at, torch, dev):
    """Inputs in HBM and a no-argument call of one leg: (fn, workload, info)."""
    from aware_tiling_amd.inputs import WORKLOADS, workload_inputs

    if leg == "headline":
        w = WORKLOADS[HEADLINE]
        q, k, v = (t.to(dev) for t in workload_inputs(w))
        o = torch.empty((w.bh, w.n, w.d), dtype=torch.float32, device=dev)
        lse = torch.empty((w.bh, w.n), dtype=torch.float32, device=dev)
        return (lambda: at.attn_fwd(q, k, v, w.scale, out=o, lse=lse)), w, {}
    if leg == "smallcache":
        w = WORKLOADS["smallcache_bf16_b1h8_n4096_d256"]
        q, k, v = (t.to(dev) for t in workload_inputs(w))
        o = torch.empty((w.bh, w.n, w.d), dtype=torch.float32, device=dev)
        lse = torch.empty((w.bh, w.n), dtype=torch.float32, device=dev)
        need = int(at.lib().attn_fwd_smallcache_workspace_size(w.bh, w.n, w.d, SMALLCACHE_M))
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        return (lambda: at.attn_fwd_smallcache(q, k, v, SMALLCACHE_M, w.scale, out=o, lse=lse,
                                               workspace=ws)), w, {"m_elems": SMALLCACHE_M,
                                                                   "q": q, "k": k, "v": v,
                                                                   "o": o, "lse": lse}
    if leg in BLOCKWISE_BWD:
        w = WORKLOADS[BLOCKWISE_BWD[leg]]
        q, k, v, do = (t.to(dev) for t in workload_inputs(w))
        o, lse = at.attn_fwd(q, k, v, w.scale)
        grads = tuple(torch.empty((w.bh, w.n, w.d), dtype=torch.float32, device=dev)
                      for _ in range(3))
        need = int(at.lib().attn_bwd_workspace_size(w.bh, w.n, w.d))
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        return (lambda: at.attn_bwd(q, k, v, o, do, lse, w.scale, workspace=ws, grads=grads)), w, \
            {"m_elems": at.bwd_onchip_elems(w.d)}
    if leg in SMALLCACHE_BWD:
        name, m_sc = SMALLCACHE_BWD[leg]
        w = WORKLOADS[name]
        q, k, v, do = (t.to(dev) for t in workload_inputs(w))
        o, lse = at.attn_fwd(q, k, v, w.scale)
        grads = tuple(torch.empty((w.bh, w.n, w.d), dtype=torch.float32, device=dev)
                      for _ in range(3))
        need = int(at.lib().attn_bwd_smallcache_workspace_size(w.bh, w.n, w.d, m_sc))
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        return (lambda: at.attn_bwd_smallcache(q, k, v, o, do, lse, m_sc, w.scale, workspace=ws,
                                               grads=grads)), w, {"m_elems": m_sc}
    raise SystemExit(f"unknown leg {leg}")


def profile_leg(leg: str, calls: int, at, torch, dev):
    """One warm call and `calls` more of one leg, for a counter run: the
    counters of the leg's kernels summed over all dispatches, divided by
    calls + 1, give its bytes per call."""
    fn, w, _ = leg_call(leg, at, torch, dev)
    torch.cuda.synchronize()
    for _ in range(calls + 1):
        fn()
    torch.cuda.synchronize()
    print(json.dumps({"leg": leg, "workload": w.name, "calls": calls + 1}), flush=True)


def summarize_leg_counters(pmc_dir: str, out_path: str = TRAFFIC_FILE):
    """HBM bytes per call of each profiled leg from rocprofv3 --pmc CSVs:
    <dir>/<leg>_fetch_counter_collection.csv and <leg>_write_..., taken on
    `--profile-leg <leg> --calls C`, and copyfetch_ / copywrite_ taken on
    `--calibrate-copy`.  Each counter (KiB per dispatch) is scaled by what it
    reads for a plain copy of COPY_BYTES."""
    import csv

    def total(fname, counter, subs):
        tot, disp = 0.0, 0
        with open(os.path.join(pmc_dir, fname)) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter and any(x in r["Kernel_Name"] for x in subs):
                    tot += float(r["Counter_Value"])
                    disp += 1
        return tot, disp

    cf = copy_counter(os.path.join(pmc_dir, "copyfetch_counter_collection.csv"), "FETCH_SIZE")
    cw = copy_counter(os.path.join(pmc_dir, "copywrite_counter_collection.csv"), "WRITE_SIZE")
    rf, rw = COPY_BYTES / cf, COPY_BYTES / cw  # bytes per counter unit
    legs = {}
    for leg, (_, subs) in LEGS.items():
        fpath = os.path.join(pmc_dir, f"{leg}_fetch_counter_collection.csv")
        if not os.path.exists(fpath):
            continue
        with open(os.path.join(pmc_dir, f"{leg}_calls.json")) as f:
            calls = [json.loads(x) for x in f if x.startswith("{")][-1]["calls"]
        fe, nf = total(f"{leg}_fetch_counter_collection.csv", "FETCH_SIZE", subs)
        wr, nw = total(f"{leg}_write_counter_collection.csv", "WRITE_SIZE", subs)
        legs[leg] = {"kernel_digest": kernel_digest(leg), "calls": calls,
                     "dispatches": [nf, nw],
                     "read_bytes_per_call": round(fe * rf / calls),
                     "write_bytes_per_call": round(wr * rw / calls),
                     "bytes_per_call": round((fe * rf + wr * rw) / calls)}
    summary = {"copy_calibration": {"copy_bytes": COPY_BYTES, "fetch_size_kib": cf,
                                    "write_size_kib": cw, "bytes_per_fetch_unit": rf,
                                    "bytes_per_write_unit": rw},
               "legs": legs}
    with open(out_path, "w") as f:
        json.dump(summary, f, indent=1)
    print(json.dumps(summary))


def cpu_baseline(w, cpu_inputs, target_s: float = 15.0):
    """The float64 oracle, as it stands, on a bounded sample of the same
    workload: whole heads (all query rows, all keys), as many as fit in about
    target_s seconds, or the leading rows of head 0 if one head is more."""
    import oracle

    q, k, v = cpu_inputs
    flops_row = 4.0 * w.n * w.d
    calib = 256  # enough rows to occupy every host thread
    qd0 = q[:1, :calib].double().numpy()
    kd0, vd0 = k[:1].double().numpy(), v[:1].double().numpy()
    oracle.attn_fwd(qd0[:, :8], kd0, vd0, w.scale)  # load + warm
    t0 = time.perf_counter()
    _, _, threads = oracle.attn_fwd(qd0, kd0, vd0, w.scale)
    dt = time.perf_counter() - t0
    rows = max(calib, int(calib * target_s / max(dt, 1e-3)))
    if rows <= w.n:
        heads, nrows = 1, max(threads, (rows // threads) * threads)
    else:
        heads, nrows = min(w.bh, max(1, rows // w.n)), w.n
    qd = q[:heads, :nrows].double().numpy()
    kd, vd = k[:heads].double().numpy(), v[:heads].double().numpy()
    t0 = time.perf_counter()
    _, _, threads = oracle.attn_fwd(qd, kd, vd, w.scale)
    dt = time.perf_counter() - t0
    tflops = flops_row * heads * nrows / dt / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{heads} head(s) x {nrows} query rows x {w.n} keys of {w.name}, float64, "
                      f"{dt:.1f} s; TFLOP/s at 4*N*d flops per query row",
            "seconds": round(dt, 2),
            "full_workload_seconds_est": round(dt * w.n * w.bh / (heads * nrows), 1)}


def counter_means(path: str, counter: str, key_of) -> dict:
    """Per-dispatch mean of `counter` in a rocprofv3 counter_collection.csv,
    grouped by key_of(kernel name) (rows whose key is None are skipped)."""
    import csv
    import statistics

    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            key = key_of(r["Kernel_Name"])
            if key is not None:
                vals.setdefault(key, []).append(float(r["Counter_Value"]))
    return {k: statistics.mean(v) for k, v in vals.items()}


def copy_counter(path: str, counter: str) -> float:
    """Mean of `counter` over the calibration copies (--calibrate-copy)."""
    return counter_means(path, counter, lambda n: "copy" if "copyBuffer" in n else None)["copy"]


def fused_sweep_key(name: str):
    """(B_r, B_c) of a d = 128 direct fused-forward kernel name (demangled or
    mangled), else None."""
    import re

    m = re.search(r"fwd_fused_bf16_direct_kernel(?:<128, (\d+), (\d+),|ILi128ELi(\d+)ELi(\d+)E)",
                  name)
    if not m:
        return None
    nw, bc = (m.group(1), m.group(2)) if m.group(1) else (m.group(3), m.group(4))
    return (32 * int(nw), int(bc))


def mfma_busy(pmc_dir: str, fname: str, key_of) -> dict:
    """Matrix-core utilisation per key: SQ_VALU_MFMA_BUSY_CYCLES over the
    SIMD-cycles of the dispatch (1024 SIMDs; GRBM_GUI_ACTIVE sums the 8
    XCDs' cycles, so SIMD-cycles = 128 x GRBM_GUI_ACTIVE).  Kernels sharing a
    key (the two launches of one path) are summed before dividing.  Empty
    when the counter file is absent."""
    path = os.path.join(pmc_dir, fname)
    if not os.path.exists(path):
        return {}
    b = counter_means(path, "SQ_VALU_MFMA_BUSY_CYCLES", lambda n: (key_of(n), n) if key_of(n) else None)
    g = counter_means(path, "GRBM_GUI_ACTIVE", lambda n: (key_of(n), n) if key_of(n) else None)
    out = {}
    for (key, name), v in b.items():
        acc = out.setdefault(key, [0.0, 0.0])
        acc[0] += v
        acc[1] += g[(key, name)]
    return {k: bv / (128.0 * gv) for k, (bv, gv) in out.items() if gv > 0}


def fmt_busy(x) -> str:
    return "n/a" if x is None else f"{x:.2f}"


def summarize_sweep(pmc_dir: str, timing_path: str, out_path: str):
    """Combine the tile sweep's timing lines with its counter runs into a
    markdown table: CU<->L2 read bytes (TCC_READ_SECTORS) and L2-miss read
    bytes (FETCH_SIZE), each scaled by what the counter reads for a plain
    copy of COPY_BYTES, against the schedule-exact and the page's models.
    Expects <dir>/sweepread_, sweepfetch_, copyread_ and copyfetch_
    counter_collection.csv, and optionally sweepmfma_ (matrix-core busy)."""
    def per_tile(fname, counter):
        return counter_means(os.path.join(pmc_dir, fname), counter, fused_sweep_key)

    def copy_value(fname, counter):
        return copy_counter(os.path.join(pmc_dir, fname), counter)

    rd = per_tile("sweepread_counter_collection.csv", "TCC_READ_SECTORS_sum")
    fe = per_tile("sweepfetch_counter_collection.csv", "FETCH_SIZE")
    busy = mfma_busy(pmc_dir, "sweepmfma_counter_collection.csv", fused_sweep_key)
    rd_unit = COPY_BYTES / copy_value("copyread_counter_collection.csv", "TCC_READ_SECTORS_sum")
    fe_unit = COPY_BYTES / copy_value("copyfetch_counter_collection.csv", "FETCH_SIZE")
    rows = [json.loads(line) for line in open(timing_path) if line.startswith("{")]
    compulsory = 402653184  # Q, K, V once (bf16)
    lines = ["| tile | B_r | B_c | M (elements) | ms | TFLOP/s | CU->L2 read bytes | "
             "schedule 2N^2d/B_r+Nd | ratio | page N^2d^2/M+Nd | ratio | L2-miss read bytes "
             "| / compulsory | matrix core busy |", "|" + "---|" * 14]
    for r in rows:
        key = (r["block_rows"], r["key_tile"])
        cu = rd.get(key, float("nan")) * rd_unit
        miss = fe.get(key, float("nan")) * fe_unit
        lines.append(
            f"| {r['tile']} | {r['block_rows']} | {r['key_tile']} | {r['onchip_elems']:,} | "
            f"{r['ms']} | {r['tflops']} | {cu / 1e9:.2f} GB | {r['sched_read_bytes'] / 1e9:.2f} GB | "
            f"{cu / r['sched_read_bytes']:.3f} | {r['page_model_bytes'] / 1e9:.2f} GB | "
            f"{cu / r['page_model_bytes']:.3f} | {miss / 1e9:.3f} GB | {miss / compulsory:.2f} | "
            f"{fmt_busy(busy.get(key))} |")
    text = "\n".join(lines) + "\n"
    text += (f"\nCounter scaling: one TCC_READ_SECTORS unit = {rd_unit:.2f} bytes and one "
             f"FETCH_SIZE unit = {fe_unit:.1f} bytes (a plain copy of {COPY_BYTES} bytes).\n")
    with open(out_path, "w") as f:
        f.write(text)
    print(text)


def smallcache_sweep_key(name: str):
    """Tile b of a d = 256 small-cache forward kernel name (demangled or
    mangled), else None."""
    import re

    m = re.search(r"sc_(?:scores_exp|value_product)(?:<256, (\d+)>|ILi256ELi(\d+)E)", name)
    return int(m.group(1) or m.group(2)) if m else None


def summarize_smallcache_sweep(pmc_dir: str, timing_path: str, out_path: str):
    """Markdown table of the small-cache tile sweep: per tile b, the two
    kernels' CU->L2 read bytes (TCC_READ_SECTORS), L2-miss read and write
    bytes (FETCH_SIZE, WRITE_SIZE) and matrix-core busy, against the
    square-tile schedule's exact panel count and the page's N^2 d / sqrt(M)
    model.  Expects <dir>/scread_, scfetch_, scwrite_, scmfma_, copyread_,
    copyfetch_ and copywrite_ counter_collection.csv."""
    def per_kernel(fname, counter):
        # mean per dispatch of each kernel: {(b, is_value_product): mean}
        return counter_means(os.path.join(pmc_dir, fname), counter,
                             lambda n: (smallcache_sweep_key(n), "value" in n)
                             if smallcache_sweep_key(n) else None)

    def sums(fname, counter):
        # summed over the two kernels of a b
        out = {}
        for (b, _), v in per_kernel(fname, counter).items():
            out[b] = out.get(b, 0.0) + v
        return out

    cu = sums("scread_counter_collection.csv", "TCC_READ_SECTORS_sum")
    cu_k = per_kernel("scread_counter_collection.csv", "TCC_READ_SECTORS_sum")
    fe = sums("scfetch_counter_collection.csv", "FETCH_SIZE")
    wr = sums("scwrite_counter_collection.csv", "WRITE_SIZE")
    busy = mfma_busy(pmc_dir, "scmfma_counter_collection.csv", smallcache_sweep_key)
    rd_unit = COPY_BYTES / copy_counter(os.path.join(pmc_dir, "copyread_counter_collection.csv"),
                                        "TCC_READ_SECTORS_sum")
    fe_unit = COPY_BYTES / copy_counter(os.path.join(pmc_dir, "copyfetch_counter_collection.csv"),
                                        "FETCH_SIZE")
    wr_unit = COPY_BYTES / copy_counter(os.path.join(pmc_dir, "copywrite_counter_collection.csv"),
                                        "WRITE_SIZE")
    rows = [json.loads(line) for line in open(timing_path) if line.startswith("{")]
    lines = ["| b | M (elements) | ms | TFLOP/s | CU->L2 read bytes | schedule 4N^2d/b | ratio | "
             "page N^2d/sqrt(M)+Nd | ratio | L2-miss read bytes | L2-miss write bytes | "
             "E round trip 2N^2 | matrix core busy |", "|" + "---|" * 13]
    for r in rows:
        b = r["tile_b"]
        c = cu.get(b, float("nan")) * rd_unit
        lines.append(
            f"| {b} | {r['onchip_elems']:,} | {r['ms']} | {r['tflops']} | {c / 1e9:.2f} GB | "
            f"{r['sched_read_bytes'] / 1e9:.2f} GB | {c / r['sched_read_bytes']:.3f} | "
            f"{r['page_model_bytes'] / 1e9:.3f} GB | {c / r['page_model_bytes']:.2f} | "
            f"{fe.get(b, float('nan')) * fe_unit / 1e9:.3f} GB | "
            f"{wr.get(b, float('nan')) * wr_unit / 1e9:.3f} GB | {r['exp_matrix_bytes'] / 1e9:.3f} GB | "
            f"{fmt_busy(busy.get(b))} |")
    lines += ["", "Per kernel, CU->L2 read bytes against its half of the schedule "
              "(2 N^2 d / b bf16 elements per head each: the scores read a b x d panel of Q "
              "and of K per tile, the value product a b x N panel of E and an N x b panel "
              "of V per output tile):", "",
              "| b | sc_scores_exp | its schedule | ratio | sc_value_product | its schedule | "
              "ratio |", "|" + "---|" * 7]
    for r in rows:
        b = r["tile_b"]
        half = r["sched_read_bytes"] / 2
        sc = cu_k.get((b, False), float("nan")) * rd_unit
        vp = cu_k.get((b, True), float("nan")) * rd_unit
        lines.append(f"| {b} | {sc / 1e9:.3f} GB | {half / 1e9:.3f} GB | {sc / half:.3f} | "
                     f"{vp / 1e9:.3f} GB | {half / 1e9:.3f} GB | {vp / half:.3f} |")
    text = "\n".join(lines) + "\n"
    text += (f"\nCounter scaling: one TCC_READ_SECTORS unit = {rd_unit:.2f} bytes, one FETCH_SIZE "
             f"unit = {fe_unit:.1f} bytes, one WRITE_SIZE unit = {wr_unit:.1f} bytes (a plain "
             f"copy of {COPY_BYTES} bytes).\n")
    with open(out_path, "w") as f:
        f.write(text)
    print(text)



def bwd_sweep_key(name: str):
    """("dkdv", waves) or ("dq", waves, key tile) of a d = 128 blockwise
    backward kernel name (demangled or mangled), else None."""
    import re

    m = re.search(r"bwd_dkdv3(?:<128, (\d+)>|ILi128ELi(\d+)E)", name)
    if m:
        return ("dkdv", int(m.group(1) or m.group(2)))
    m = re.search(r"bwd_dq3(?:<128, (\d+), (\d+)>|ILi128ELi(\d+)ELi(\d+)E)", name)
    if m:
        nw, bc = (m.group(1), m.group(2)) if m.group(1) else (m.group(3), m.group(4))
        return ("dq", int(nw), int(bc))
    return None


def summarize_bwd_sweep(pmc_dir: str, timing_path: str, out_path: str):
    """Markdown table of the blockwise backward's tile sweep: per shape, the
    dK/dV and dQ kernels' CU->L2 read bytes (TCC_READ_SECTORS) and L2-miss
    read bytes (FETCH_SIZE), scaled by a plain copy, against the schedule's
    count, and the two kernels' matrix-core busy fraction.  Expects
    <dir>/bwdread_, bwdfetch_, bwdmfma_, copyread_ and copyfetch_
    counter_collection.csv."""
    def means(fname, counter):
        return counter_means(os.path.join(pmc_dir, fname), counter, bwd_sweep_key)

    cu = means("bwdread_counter_collection.csv", "TCC_READ_SECTORS_sum")
    fe = means("bwdfetch_counter_collection.csv", "FETCH_SIZE")
    busy_c = means("bwdmfma_counter_collection.csv", "SQ_VALU_MFMA_BUSY_CYCLES")
    grbm = means("bwdmfma_counter_collection.csv", "GRBM_GUI_ACTIVE")
    rd_unit = COPY_BYTES / copy_counter(os.path.join(pmc_dir, "copyread_counter_collection.csv"),
                                        "TCC_READ_SECTORS_sum")
    fe_unit = COPY_BYTES / copy_counter(os.path.join(pmc_dir, "copyfetch_counter_collection.csv"),
                                        "FETCH_SIZE")
    rows = [json.loads(line) for line in open(timing_path) if line.startswith("{")]
    lines = ["| tile | keys per dK/dV block | queries per dQ block | keys per dQ tile | "
             "M (elements) | ms | TFLOP/s at 10N^2d | CU->L2 read bytes | schedule | ratio | "
             "L2-miss read bytes | matrix core busy |", "|" + "---|" * 12]
    for r in rows:
        ks = (("dkdv", r["keys_per_block"] // 32),
              ("dq", r["queries_per_block"] // 32, r["key_tile"]))
        c = sum(cu.get(x, float("nan")) for x in ks) * rd_unit
        f = sum(fe.get(x, float("nan")) for x in ks) * fe_unit
        cyc = sum(grbm.get(x, float("nan")) for x in ks) / 8.0
        busy = sum(busy_c.get(x, float("nan")) for x in ks) / (1024.0 * cyc)
        lines.append(
            f"| {r['tile']} | {r['keys_per_block']} | {r['queries_per_block']} | {r['key_tile']} | "
            f"{r['onchip_elems']:,} | {r['ms']} | {r['tflops_at_10N2d']} | {c / 1e9:.2f} GB | "
            f"{r['sched_read_bytes'] / 1e9:.2f} GB | {c / r['sched_read_bytes']:.3f} | "
            f"{f / 1e9:.3f} GB | {fmt_busy(busy)} |")
    text = "\n".join(lines) + "\n"
    text += (f"\nCounter scaling: one TCC_READ_SECTORS unit = {rd_unit:.2f} bytes and one "
             f"FETCH_SIZE unit = {fe_unit:.1f} bytes (a plain copy of {COPY_BYTES} bytes).\n")
    with open(out_path, "w") as f:
        f.write(text)
    print(text)


def bwd_tile_sweep(args, at, torch, dev):
    """Time the blockwise backward at every compiled tile shape (d = 128) on
    the backward workload; one JSON line per shape."""
    fn, w, info = leg_call("backward", at, torch, dev)
    del fn
    from aware_tiling_amd.inputs import workload_inputs

    q, k, v, do = (t.to(dev) for t in workload_inputs(w))
    o, lse = at.attn_fwd(q, k, v, w.scale)
    grads = tuple(torch.empty((w.bh, w.n, w.d), dtype=torch.float32, device=dev)
                  for _ in range(3))
    need = int(at.lib().attn_bwd_workspace_size(w.bh, w.n, w.d))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    fl = 10.0 * w.n * w.n * w.d * w.bh
    for name in at.bwd_tiles(w.d):
        t = at.bwd_tile_info(name, w.d)
        print(f"[bench] backward tile {name}", file=sys.stderr, flush=True)
        ms, _, _ = time_launches(lambda: at.attn_bwd_tile(name, q, k, v, o, do, lse, w.scale,
                                                          workspace=ws, grads=grads),
                                 args.steps, args.warmup, batch=True, warm_s=SECONDARY_WARM_S)
        # CU->L2 reads of the schedule, bf16: every dK/dV block reads all of Q
        # and dO (and its own K, V rows once); every dQ block all of K and V
        # (and its own Q, dO rows once)
        nd2 = w.n * w.d * 2
        sched = w.bh * (2 * nd2 * (-(-w.n // t["keys_per_block"])) + 2 * nd2 +
                        2 * nd2 * (-(-w.n // t["queries_per_block"])) + 2 * nd2)
        print(json.dumps({"tile": name, **t, "ms": round(ms, 4),
                          "tflops_at_10N2d": round(fl / (ms * 1e-3) / 1e12, 2),
                          "sched_read_bytes": sched}), flush=True)

def main():
    if len(sys.argv) >= 5 and sys.argv[1] == "--summarize-smallcache-sweep":
        summarize_smallcache_sweep(sys.argv[2], sys.argv[3], sys.argv[4])
        return
    if len(sys.argv) >= 3 and sys.argv[1] == "--summarize-leg-counters":
        summarize_leg_counters(sys.argv[2])
        return
    if len(sys.argv) >= 5 and sys.argv[1] == "--summarize-bwd-sweep":
        summarize_bwd_sweep(sys.argv[2], sys.argv[3], sys.argv[4])
        return
    if len(sys.argv) >= 5 and sys.argv[1] == "--summarize-sweep":
        summarize_sweep(sys.argv[2], sys.argv[3], sys.argv[4])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--legs", default=None,
                    help="comma-separated secondary legs to run (smallcache, backward, "
                         "smallcache_backward, blocksparse, splitk); default all")
    ap.add_argument("--secondary-only", action="store_true",
                    help="skip the headline and print only the secondary legs' JSON")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="time every query-block x key-tile shape of the fused forward on the "
                         "headline workload (one JSON line per shape) and exit")
    ap.add_argument("--bwd-tile-sweep", action="store_true",
                    help="time the blockwise backward at every compiled tile shape (d = 128) "
                         "on the backward workload (one JSON line per shape) and exit")
    ap.add_argument("--smallcache-sweep", action="store_true",
                    help="time the square-tile forward at every tile b on the d = 256 "
                         "small-cache workload (one JSON line per tile) and exit")
    ap.add_argument("--profile-leg", default=None, choices=sorted(LEGS),
                    help="run one leg --calls + 1 times (for a counter run) and exit")
    ap.add_argument("--calls", type=int, default=3)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 1 GiB three times (to scale the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (heads are "
              "independent, so a multi-GPU run would shard batch x heads with no communication)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import aware_tiling_amd as at
    from aware_tiling_amd.inputs import WORKLOADS, workload_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 3}))
        return
    if args.profile_leg:
        profile_leg(args.profile_leg, args.calls, at, torch, dev)
        return
    if args.tile_sweep:
        tile_sweep(args, at, torch, dev)
        return
    if args.smallcache_sweep:
        smallcache_sweep(args, at, torch, dev)
        return
    if args.bwd_tile_sweep:
        bwd_tile_sweep(args, at, torch, dev)
        return
    if args.secondary_only:
        print(json.dumps({"secondary": secondary(args, at, torch, dev)}), flush=True)
        return
    w = WORKLOADS[HEADLINE]
    print(f"[bench] inputs {w.name}", file=sys.stderr, flush=True)
    cpu_inputs = workload_inputs(w)
    q, k, v = (t.to(dev) for t in cpu_inputs)
    o = torch.empty((w.bh, w.n, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.bh, w.n), dtype=torch.float32, device=dev)
    fn = lambda: at.attn_fwd(q, k, v, w.scale, out=o, lse=lse)
    print(f"[bench] timing attn_fwd steps={args.steps} warmup={args.warmup}", file=sys.stderr,
          flush=True)
    torch.cuda.synchronize()
    launch_ms, wall_ms, ev = time_launches(fn, args.steps, args.warmup)
    flops = w.fwd_flops
    tflops = flops / (wall_ms * 1e-3) / 1e12
    achieved = flops / (launch_ms * 1e-3) / 1e12
    compulsory = w.bh * (3 * w.n * w.d * 2 + w.n * w.d * 4 + w.n * 4)
    br = at.fwd_query_block(w.d)
    m_elems = at.fwd_onchip_elems(w.d)
    # the exposition's fused-schedule models, in bytes (bf16 inputs)
    sched_bytes = w.bh * (2 * w.n * w.n * w.d / br + 2 * w.n * w.d) * 2
    model_bytes = w.bh * (w.n * w.n * w.d * w.d / m_elems + w.n * w.d) * 2

    traffic = traffic_for_launch()
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "kernel": "attn_fwd fused kernel (default tile, d=128)",
                "flops_per_launch": flops, "launch_ms": round(launch_ms, 4)}
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq_len": w.n,
                   "head_dim": w.d, "q_scale": w.q_mult, "query_block": br,
                   "onchip_elems": m_elems, "tile": at.fwd_tiles(w.d)[0]},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "hbm_gbps": round(compulsory / (wall_ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(compulsory / (wall_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "bytes": {"compulsory": compulsory, "fused_schedule_cu_boundary": sched_bytes,
                  "page_model_N2d2_over_M_plus_Nd": model_bytes},
        "roofline": roofline,
        "launch_ms_min": round(min(ev), 4),
        "launch_ms_max": round(max(ev), 4),
        "launch_ms_median": round(percentile(ev, 50), 4),
        "launch_ms_p90": round(percentile(ev, 90), 4),
    }
    if traffic:
        out["l2miss_gbps"] = round(traffic / (launch_ms * 1e-3) / 1e9, 1)
    out["cold_launch_ms"] = round(cold_launch_ms(fn, torch, dev), 4)
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    out["measured_peaks"] = measured_peaks(torch, dev, at)
    out["frac_of_measured_gemm"] = round(achieved / out["measured_peaks"]["gemm_bf16_tflops"], 4)
    out["frac_of_measured_mfma_loop"] = round(
        achieved / out["measured_peaks"]["mfma_loop_bf16_tflops"], 4)

    if not args.no_secondary:
        out["secondary"] = secondary(args, at, torch, dev)
        dec = out["secondary"].get("splitk_decode")
        if dec is not None and "stream_read_gbps" in out["measured_peaks"]:
            dec["frac_of_measured_stream_read"] = round(
                dec["hbm_gbps"] / out["measured_peaks"]["stream_read_gbps"], 4)

    if not args.no_cpu:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, cpu_inputs)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


SWEEP_TILES = ["r64c32", "r64c64", "r128c32", "r128c64", "r256c32", "r256c64"]


def tile_sweep(args, at, torch, dev):
    """The fused forward at B_r in {64, 128, 256} query rows and B_c in
    {32, 64} keys per tile, on the headline workload: time and the byte
    models of each shape (the counters come from rocprofv3 runs of this
    same mode; see --summarize-sweep)."""
    from aware_tiling_amd.inputs import WORKLOADS, workload_inputs

    w = WORKLOADS[HEADLINE]
    q, k, v = (t.to(dev) for t in workload_inputs(w))
    o = torch.empty((w.bh, w.n, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.bh, w.n), dtype=torch.float32, device=dev)
    for name in SWEEP_TILES:
        info = at.fwd_tile_info(name, w.d)
        br, m_elems = info["block_rows"], info["onchip_elems"]
        print(f"[bench] tile {name}", file=sys.stderr, flush=True)
        ms, _, _ = time_launches(lambda: at.attn_fwd_tile(name, q, k, v, w.scale, out=o, lse=lse),
                                 args.steps, args.warmup)
        # per launch, in bytes (bf16 K/V stream + Q once); elements x 2
        sched = w.bh * (2 * w.n * w.n * w.d / br + w.n * w.d) * 2
        model = w.bh * (w.n * w.n * w.d * w.d / m_elems + w.n * w.d) * 2
        print(json.dumps({"tile": name, "block_rows": br, "key_tile": info["key_tile"],
                          "onchip_elems": m_elems, "ms": round(ms, 4),
                          "tflops": round(w.fwd_flops / (ms * 1e-3) / 1e12, 1),
                          "sched_read_bytes": sched, "page_model_bytes": model}), flush=True)


SC_SWEEP_B = (128, 64)


def smallcache_sweep(args, at, torch, dev):
    """The square-tile forward at each tile b, with M set to that tile's
    exact on-chip footprint, on the d = 256 small-cache workload: time and
    the byte models (counters from rocprofv3 runs of this same mode; see
    --summarize-smallcache-sweep)."""
    from aware_tiling_amd.inputs import WORKLOADS, workload_inputs

    w = WORKLOADS["smallcache_bf16_b1h8_n4096_d256"]
    q, k, v = (t.to(dev) for t in workload_inputs(w))
    o = torch.empty((w.bh, w.n, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.bh, w.n), dtype=torch.float32, device=dev)
    for b in SC_SWEEP_B:
        m_elems = int(at.lib().attn_smallcache_onchip_elems(b))
        if m_elems <= 0 or at.smallcache_tile(w.d, m_elems) != b:
            raise RuntimeError(f"tile b={b} is not selected at its own footprint {m_elems}")
        need = int(at.lib().attn_fwd_smallcache_workspace_size(w.bh, w.n, w.d, m_elems))
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        print(f"[bench] small-cache tile b={b} M={m_elems}", file=sys.stderr, flush=True)
        ms, _, _ = time_launches(lambda: at.attn_fwd_smallcache(
            q, k, v, m_elems, w.scale, out=o, lse=lse, workspace=ws), args.steps, args.warmup,
            batch=True, warm_s=SECONDARY_WARM_S)
        # per launch, bytes: every (query tile, key tile) reads a b x d panel of Q
        # and of K; every (query tile, b-wide output column block) reads a
        # b x N panel of E and an N x b panel of V -- 4 N^2 d / b bf16 elements
        sched = w.bh * 4 * w.n * w.n * w.d / b * 2
        model = w.bh * (w.n * w.n * w.d / math.sqrt(m_elems) + w.n * w.d) * 2
        print(json.dumps({"tile_b": b, "onchip_elems": m_elems, "ms": round(ms, 4),
                          "tflops": round(w.fwd_flops / (ms * 1e-3) / 1e12, 1),
                          "sched_read_bytes": sched, "page_model_bytes": model,
                          "exp_matrix_bytes": w.bh * 2 * w.n * w.n * 2}), flush=True)
        del ws


def theorem_1_1(w, m: int) -> dict:
    """Theorem 1.1 of the page "On Fine-Grained I/O Complexity of Attention
    Backward Passes": Theta(min((n^2 d^2 + n d^3) / M, (n^2 d + n d^2) /
    sqrt(M))) transfers per head, evaluated without its constant (elements,
    reported as bf16 bytes) -- a model, not a pinned parity."""
    n, d = w.n, w.d
    large = (n * n * d * d + n * d ** 3) / m
    small = (n * n * d + n * d * d) / math.sqrt(m)
    return {"name": "theorem_1_1", "regime": "large-cache (M >= d^2)" if m >= d * d
            else "small-cache (M < d^2)", "m_elems": m,
            "elements": round(w.bh * min(large, small)), "bytes": round(2 * w.bh * min(large, small))}


def page_fwd_smallcache(w, m: int) -> dict:
    """The exposition's N^2 d / sqrt(M) + N d movement for the square-tile
    forward (table under "Putting the regimes together"), per head, as bf16
    bytes -- a model without its constant."""
    el = w.n * w.n * w.d / math.sqrt(m) + w.n * w.d
    return {"name": "N^2 d / sqrt(M) + N d", "m_elems": m, "elements": round(w.bh * el),
            "bytes": round(2 * w.bh * el)}


def leg_bytes(leg: str, ms: float, floor_bytes: float, model: dict,
              with_roofline: bool = True) -> dict:
    """HBM bytes of one call of a leg from the committed counter summary
    (None when it was taken on other kernel sources), their ratio to the
    page's model, and (with_roofline) the leg's roofline against its HBM
    floor: floor_bytes / 8 TB/s over the measured time."""
    t = leg_traffic(leg)
    out = {"hbm_floor_bytes": round(floor_bytes), "model": model,
           "counter_bytes": t["bytes_per_call"] if t else None,
           "counter_read_bytes": t["read_bytes_per_call"] if t else None,
           "counter_write_bytes": t["write_bytes_per_call"] if t else None,
           "counter_to_model": round(t["bytes_per_call"] / model["bytes"], 3) if t else None}
    if with_roofline:
        gbps = floor_bytes / (ms * 1e-3) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                           "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                           "what": "HBM floor bytes / measured time"}
    return out


def secondary(args, at, torch, dev):
    from aware_tiling_amd.inputs import WORKLOADS, workload_inputs

    res = {}
    legs = set(args.legs.split(",")) if args.legs else None

    def want(name):
        return legs is None or name in legs

    if want("smallcache") and at.smallcache_tile(256, SMALLCACHE_M) > 0:
        fn, w, info = leg_call("smallcache", at, torch, dev)
        print(f"[bench] timing {w.name}", file=sys.stderr, flush=True)
        q, k, v, o, lse = (info[x] for x in ("q", "k", "v", "o", "lse"))
        m_elems = info["m_elems"]
        ms_sc, _, _ = time_launches(fn, args.steps, args.warmup, batch=True,
                                    warm_s=SECONDARY_WARM_S)
        ms_fu, _, _ = time_launches(lambda: at.attn_fwd(q, k, v, w.scale, out=o, lse=lse),
                                    args.steps, args.warmup, batch=True, warm_s=SECONDARY_WARM_S)
        b = at.smallcache_tile(w.d, m_elems)
        # HBM floor: Q, K, V read and O, lse written once, and the exponentiated
        # matrix E written once and read once (bf16)
        e_bytes = w.bh * w.n * w.n * 2
        floor = w.bh * (3 * w.n * w.d * 2 + w.n * w.d * 4 + w.n * 4) + 2 * e_bytes
        res["smallcache"] = {"workload": w.name, "m_elems": m_elems, "tile_b": b,
                             "onchip_elems": int(at.lib().attn_smallcache_onchip_elems(b)),
                             "ms": round(ms_sc, 4),
                             "tflops": round(w.fwd_flops / (ms_sc * 1e-3) / 1e12, 2),
                             "fused_ms_same_inputs": round(ms_fu, 4),
                             "fused_tflops": round(w.fwd_flops / (ms_fu * 1e-3) / 1e12, 2),
                             "exp_matrix_bytes": e_bytes,
                             **leg_bytes("smallcache", ms_sc, floor, page_fwd_smallcache(w, m_elems))}
        # both schedules held to the same budget below d^2: the fused one with
        # 32-row query blocks (K, V read once per block) and the square tiles
        m_same = at.fwd_budget_onchip_elems(w.d)
        if m_same > 0 and at.smallcache_tile(w.d, m_same) > 0:
            need = int(at.lib().attn_fwd_smallcache_workspace_size(w.bh, w.n, w.d, m_same))
            ws2 = torch.empty(need, dtype=torch.uint8, device=dev)
            ms_fb, _, _ = time_launches(lambda: at.attn_fwd_budget(
                q, k, v, m_same, w.scale, out=o, lse=lse), args.steps, args.warmup, batch=True,
                warm_s=SECONDARY_WARM_S)
            ms_sb, _, _ = time_launches(lambda: at.attn_fwd_smallcache(
                q, k, v, m_same, w.scale, out=o, lse=lse, workspace=ws2), args.steps,
                args.warmup, batch=True, warm_s=SECONDARY_WARM_S)
            res["smallcache"]["same_budget"] = {
                "m_elems": m_same,
                "fused_query_rows": 32, "fused_ms": round(ms_fb, 4),
                "fused_tflops": round(w.fwd_flops / (ms_fb * 1e-3) / 1e12, 2),
                "fused_kv_bytes": w.bh * (w.n // 32) * 2 * w.n * w.d * 2,
                "smallcache_tile_b": at.smallcache_tile(w.d, m_same),
                "smallcache_ms": round(ms_sb, 4),
                "smallcache_tflops": round(w.fwd_flops / (ms_sb * 1e-3) / 1e12, 2)}
            del ws2
        del fn, info, q, k, v, o, lse
        torch.cuda.empty_cache()
    for leg in (BLOCKWISE_BWD if want("backward") else ()):
        fn, w, info = leg_call(leg, at, torch, dev)
        print(f"[bench] timing blockwise backward {w.name}", file=sys.stderr, flush=True)
        ms, _, _ = time_launches(fn, args.steps, args.warmup, batch=True, warm_s=SECONDARY_WARM_S)
        fl = 10.0 * w.n * w.n * w.d * w.bh  # five n x n x d products, 2 n^2 d flops each
        m = info["m_elems"]
        # HBM floor: Q, K, V, dO (bf16), O, lse read, dQ, dK, dV (fp32) written
        floor = w.bh * (4 * w.n * w.d * 2 + w.n * w.d * 4 + w.n * 4 + 3 * w.n * w.d * 4)
        res[leg] = {
            "workload": w.name, "ms": round(ms, 4), "onchip_elems": m,
            "tflops_at_10N2d": round(fl / (ms * 1e-3) / 1e12, 2),
            "roofline": {"bound": "mfma", "achieved": round(fl / (ms * 1e-3) / 1e12, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
            **leg_bytes(leg, ms, floor, theorem_1_1(w, m), with_roofline=False)}
        del fn, info
        torch.cuda.empty_cache()
    for leg in (SMALLCACHE_BWD if want("smallcache_backward") else ()):
        fn, w, info = leg_call(leg, at, torch, dev)
        m_sc = info["m_elems"]
        b = at.bwd_smallcache_tile(w.d, m_sc)
        print(f"[bench] timing small-cache backward {w.name} M={m_sc}", file=sys.stderr,
              flush=True)
        ms, _, _ = time_launches(fn, args.steps, args.warmup, batch=True, warm_s=SECONDARY_WARM_S)
        npad = -(-w.n // b) * b
        fl = 10.0 * w.n * w.n * w.d * w.bh
        # n x n traffic of the schedule: P^T and dS^T written once, P^T read
        # once (dV), dS^T read twice (dK, dQ); bf16
        nn_bytes = 5 * w.bh * npad * npad * 2
        # HBM floor: that n x n traffic and the backward's own inputs and outputs
        floor = nn_bytes + w.bh * (4 * w.n * w.d * 2 + w.n * w.d * 4 + w.n * 4 +
                                   3 * w.n * w.d * 4)
        res[leg] = {
            "workload": w.name, "m_elems": m_sc, "tile_b": b,
            "onchip_elems": int(at.lib().attn_bwd_smallcache_onchip_elems(w.d, m_sc)),
            "ms": round(ms, 4), "tflops_at_10N2d": round(fl / (ms * 1e-3) / 1e12, 2),
            "nxn_bytes": nn_bytes,
            "nxn_gbps": round(nn_bytes / (ms * 1e-3) / 1e9, 1),
            **leg_bytes(leg, ms, floor, theorem_1_1(w, m_sc))}
        del fn, info
        torch.cuda.empty_cache()
    from aware_tiling_amd.inputs import make_block_mask

    if want("blocksparse"):
        w = WORKLOADS["sparse_bf16_b1h32_n16384_d128_keep25"]
        print(f"[bench] timing {w.name}", file=sys.stderr, flush=True)
        q, k, v = (t.to(dev) for t in workload_inputs(w))
        nb = -(-w.n // at.SPARSE_BLOCK)
        mask = make_block_mask(w.bh, nb, w.density, w.seed + 1000).to(dev)
        o = torch.empty((w.bh, w.n, w.d), dtype=torch.float32, device=dev)
        lse = torch.empty((w.bh, w.n), dtype=torch.float32, device=dev)
        need = int(at.lib().attn_fwd_blocksparse_workspace_size(w.bh, w.n, w.bh))
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        ms, _, _ = time_launches(lambda: at.attn_fwd_blocksparse(q, k, v, mask, w.scale, out=o,
                                                                 lse=lse, workspace=ws),
                                 args.steps, args.warmup, batch=True, warm_s=SECONDARY_WARM_S)
        ms_dense, _, _ = time_launches(lambda: at.attn_fwd(q, k, v, w.scale, out=o, lse=lse),
                                       args.steps, args.warmup, batch=True, warm_s=SECONDARY_WARM_S)
        # kept query-key pairs: per kept block, its valid queries x valid keys
        sizes = torch.full((nb,), at.SPARSE_BLOCK, dtype=torch.float64)
        sizes[-1] = w.n - (nb - 1) * at.SPARSE_BLOCK
        pairs = float(torch.einsum("hij,i,j->", mask.cpu().double(), sizes, sizes))
        fl = 4.0 * w.d * pairs
        kept = float(mask.float().mean())
        res["blocksparse"] = {
            "workload": w.name, "kept_block_fraction": round(kept, 4), "ms": round(ms, 4),
            "tflops_on_kept_pairs": round(fl / (ms * 1e-3) / 1e12, 2),
            "dense_ms_same_inputs": round(ms_dense, 4),
            "time_fraction_of_dense": round(ms / ms_dense, 4)}
        del q, k, v, o, lse, ws, mask
    for name in (("decode_bf16_b8h32_q1_k16384_d128", "chunk_bf16_b1h32_q1024_k16384_d128")
                 if want("splitk") else ()):
        w = WORKLOADS[name]
        print(f"[bench] timing {w.name}", file=sys.stderr, flush=True)
        q, k, v = (t.to(dev) for t in workload_inputs(w))
        nq = w.queries
        o = torch.empty((w.bh, nq, w.d), dtype=torch.float32, device=dev)
        lse = torch.empty((w.bh, nq), dtype=torch.float32, device=dev)
        splits = at.splitk_splits(w.bh, nq, w.n, w.d, 0)
        need = int(at.lib().attn_fwd_splitk_workspace_size(w.bh, nq, w.n, w.d, 0))
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        ms, _, _ = time_launches(lambda: at.attn_fwd_splitk(q, k, v, 0, w.scale, out=o, lse=lse,
                                                            workspace=ws),
                                 args.steps, args.warmup, batch=True, warm_s=SECONDARY_WARM_S)
        # compulsory bytes: Q, K, V in bf16; O and lse in fp32
        byts = w.bh * (nq * w.d * 2 + 2 * w.n * w.d * 2 + nq * w.d * 4 + nq * 4)
        res[w.kind + "_" + name.split("_")[0]] = {
            "workload": w.name, "splits": splits, "ms": round(ms, 4),
            "tflops": round(w.fwd_flops / (ms * 1e-3) / 1e12, 2),
            "compulsory_bytes": byts,
            "hbm_gbps": round(byts / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
        del q, k, v, o, lse, ws
    torch.cuda.synchronize()
    return res


if __name__ == "__main__":
    main()
