#!/usr/bin/env python3
"""Benchmark of the int4 decode GEMV on one MI355X.

Default run (the headline metric): the cache-defeating stream, 32 distinct
int4 group-128 matrices K=4096 x N=14336 (976,224,256 B of codes, scales and
zero points, more than L2 + Infinity Cache) cycled at M=1.  One step is one
pass over the 32 matrices (32 gemv_q4 calls, replayed from one HIP graph).
W warm-up steps, then exactly K timed steps between two device syncs, timed
with HIP events on the stream the graph runs on.  Prints ONE JSON line.

Alongside, in the same process and in ABBA order (forward, then reversed), the
measurement method of cera 0.5.0 wgpu_gemv_bench.rs is applied to three
kernels: gemv_q4 (the metric), gemv_f32 on the same shape (the control,
4 distinct 235 MB matrices cycled) and read_reduce over 2 GiB (the measured
HBM read peak).  Each cell is a two-point difference, per_iter =
(t(2n) - t(n)) / n, which cancels every fixed per-measurement cost; a cell is
"noise" unless t(2n) >= 1.2 t(n); n is swept; the first round is discarded;
medians of >= 3 runs are reported with min and p10-p90.

Also in the default line ("block_formats" and "scan2", skipped with
--no-blocks): gemv_block on the Q4_0, Q8_0, Q4_K, Q5_K and Q6_K block formats
of the cera page at the same 4096 x 14336 stream shape and at the page's four
decode shapes, each cycling >= 1 GiB of distinct matrices; and the 2-bit
corpus scan of the Refractometer page, 65,536 vectors x 8 queries, D = 768,
cycling 64 distinct corpora; one decoder layer (hidden 896, FFN 4864) as
seven GEMVs and as four launches, cycling 64 distinct layers; and the FFN
pair 4096 -> 14336 -> 4096 at 1, 2, 4 and 8 activation rows against both the
HBM and the VALU roof ("ffn_rows").  Then
("bandwidth_sweep", skipped with --no-sweep) the Refractometer page's
bandwidth sweep: vec4 read-reduce and vec4 copy over buffers from 16 KiB to
2 GiB, the best of three workgroup counts per size, cliffs marked by the
page's 80% rule, and from them the cache class of the stream's working set;
and the fixed cost of one launch in a graph ("launch_gap_us").

Other modes:
  --blocks-only     only the block-format, scan, layer, ffn and sweep cells
                    (--block-shapes to pick)
  --pmc-workload    a short fixed sequence of dispatches for rocprofv3 --pmc
  --summarize DIR   turn rocprofv3 CSV output in DIR into a profiles/ summary
The CPU oracle is timed on a bounded sample of the same workload
(cpu_baseline: rows split over up to 16 host threads, and on one thread); it
is the only use of oracle/ here.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "int4 GEMV achieved GB/s (% of HBM peak), M=1 K=4096 N=14336 streamed"
SPEC_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published peak
PROFILES = os.path.join(ROOT, "profiles")
PMC_SUMMARY = os.path.join(PROFILES, "gemv_q4_stream_4096x14336_g128_pmc.json")
KERNEL_SOURCE = os.path.join(ROOT, "memory_bandwidth_amd", "csrc", "gemv_q4.hip")
NOISE_RATIO = 1.2


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- timing method (pure)

def two_point(t_n: float, t_2n: float, n: int) -> float:
    """Per-iteration time from timings of n and 2n iterations; fixed costs cancel."""
    return (t_2n - t_n) / n


def resolvable(t_n: float, t_2n: float, ratio: float = NOISE_RATIO) -> bool:
    """Doubling the work must lengthen the run by at least `ratio`, else the cell is noise."""
    return t_2n >= ratio * t_n and t_2n > t_n


def summarize(values: list[float]) -> dict:
    v = sorted(values)
    if not v:
        return {"median": None, "min": None, "p10": None, "p90": None, "n": 0}

    def pct(p):
        k = (len(v) - 1) * p
        lo, hi = int(k), min(int(k) + 1, len(v) - 1)
        return v[lo] + (v[hi] - v[lo]) * (k - lo)
    return {"median": statistics.median(v), "min": v[0], "p10": pct(0.1), "p90": pct(0.9),
            "n": len(v)}


def abba_orders(kernels: list[str], runs: int) -> list[list[str]]:
    """Run r uses the forward order when r is even and the reversed order when odd."""
    return [list(kernels) if r % 2 == 0 else list(reversed(kernels)) for r in range(runs)]


def sweep(timer, kernels: list[str], iters: list[int], runs: int) -> dict:
    """Two-point timing of every kernel at every n, ABBA-ordered, first round discarded.

    timer(kernel, n) -> seconds for n iterations.  Returns, per kernel, the
    per-iteration samples that were resolvable and the count of noise cells.
    """
    out = {k: {"samples": [], "noise": 0, "cells": []} for k in kernels}
    for r, order in enumerate(abba_orders(kernels, runs + 1)):
        for k in order:
            for n in iters:
                t_n = timer(k, n)
                t_2n = timer(k, 2 * n)
                if r == 0:
                    continue                      # the first round only warms up
                ok = resolvable(t_n, t_2n)
                per = two_point(t_n, t_2n, n)
                out[k]["cells"].append({"run": r, "n": n, "t_n": t_n, "t_2n": t_2n,
                                        "per_iter": per if ok else None})
                if ok and per > 0:
                    out[k]["samples"].append(per)
                else:
                    out[k]["noise"] += 1
    return out


def kernel_source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()[:16]


def traffic_from_profile(launch_bytes: int):
    """HBM bytes per gemv_q4 launch from the committed --pmc summary, or None
    when there is none or the kernel source changed since it was taken."""
    try:
        s = json.load(open(PMC_SUMMARY))
    except (OSError, ValueError):
        return None
    if s.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return s.get("gemv_q4_hbm_bytes_per_launch")


# ---------------------------------------------------------------- GPU side

class Graph:
    """A captured batch of launches replayed on the current stream."""

    def __init__(self, fn, torch):
        self.torch = torch
        fn()                                   # eager run: first touch, device check
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g):
            fn()
        torch.cuda.synchronize()

    def time(self, reps: int) -> float:
        """Seconds for `reps` back-to-back replays, by HIP events on the replay stream."""
        torch = self.torch
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            self.g.replay()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) / 1e3


def setup_stream(torch, q4, dev):
    s = wl.STREAM_SHAPE
    seed = wl.workload_seed(4)
    x = torch.from_numpy(wl.make_x(seed, 1, s.K)).to(dev)
    mats = []
    t0 = time.time()
    for i in range(wl.STREAM_MATRICES):
        d = wl.make_q4_weights(seed, s.N, s.K, s.g, s.s_lo, s.s_hi, index=i)
        mats.append({k: torch.from_numpy(v).to(dev) for k, v in d.items()})
    ys = [torch.empty((1, s.N), dtype=torch.float32, device=dev) for _ in mats]
    # dense control: four of the matrices, dequantised on the device
    wf = [q4.dequant_q4(m["wq"], m["scales"], m["zeros"], s.g, want_codes=False)[0]
          for m in mats[:wl.STREAM_F32_MATRICES]]
    yf = [torch.empty((1, s.N), dtype=torch.float32, device=dev) for _ in wf]
    n_probe = wl.PROBE_BYTES // 4
    probe = torch.empty(n_probe, dtype=torch.float32, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    probe.uniform_(0.0, 1.0, generator=gen)
    partials = torch.empty(4096, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"inputs resident in HBM ({time.time() - t0:.1f} s)")
    return {"shape": s, "x": x, "mats": mats, "ys": ys, "wf": wf, "yf": yf, "probe": probe,
            "partials": partials}


def gate(torch, q4, W):
    """Refuse to time a wrong kernel: gemv_q4 must agree with gemv_f32 on the
    device-dequantised weights within the GEMV tolerance (bound from |x|.|W|^T)."""
    s = W["shape"]
    for i in range(wl.STREAM_F32_MATRICES):
        m = W["mats"][i]
        y4 = q4.gemv_q4(W["x"], m["wq"], m["scales"], m["zeros"], s.g)
        yf = q4.gemv_f32(W["x"], W["wf"][i])
        bound = q4.gemv_f32(W["x"].abs(), W["wf"][i].abs())
        err = (y4.double() - yf.double()).abs()
        tol = 2 * (1e-4 * bound.double() + 1e-6)
        if not bool((err <= tol).all()):
            raise SystemExit(f"parity gate failed on matrix {i}: worst err/tol "
                             f"{float((err / tol).max()):.3g}")
    torch.cuda.synchronize()


CPU_THREADS_MAX = 16   # the host cores one GPU's share of the machine holds


def _oracle_rate(budget_s: float, threads: int):
    """GB/s of the oracle over whole stream matrices until `budget_s` of
    oracle time: with threads > 1 each matrix's rows are split into that many
    contiguous ranges, one oracle call per range on its own thread (the
    oracle releases the interpreter lock while it runs)."""
    import concurrent.futures
    import numpy as np
    import oracle
    s = wl.STREAM_SHAPE
    seed = wl.workload_seed(4)
    x = wl.make_x(seed, 1, s.K)
    parts = np.array_split(np.arange(s.N, dtype=np.int64), threads)
    done, t_used, times = 0, 0.0, []
    mats = []                  # generated once; past the 32nd call the stream cycles
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        while t_used < budget_s or done < 3:
            i = done % wl.STREAM_MATRICES
            if i == len(mats):
                mats.append(wl.make_q4_weights(seed, s.N, s.K, s.g, s.s_lo, s.s_hi, index=i))
            d = mats[i]
            t0 = time.perf_counter()
            if threads == 1:
                oracle.gemv_q4(x, d["wq"], d["scales"], d["zeros"], s.g)
            else:
                list(ex.map(lambda r: oracle.gemv_q4(x, d["wq"], d["scales"], d["zeros"], s.g, rows=r),
                            parts))
            times.append(time.perf_counter() - t0)
            t_used += times[-1]
            done += 1
    # the median GEMV (at least three), as the GPU figures are medians
    return wl.q4_weight_bytes(s.N, s.K, s.g) / statistics.median(times) / 1e9, done, t_used


def cpu_baseline(budget_s: float = 12.0) -> dict:
    """The oracle, as it stands, on a bounded sample of the stream workload:
    on every host core of one GPU's share (at most 16 threads) and on one."""
    threads = max(1, min(CPU_THREADS_MAX, os.cpu_count() or 1))
    v1, n1, t1 = _oracle_rate(budget_s / 2, 1)
    vn, nn, tn = _oracle_rate(budget_s / 2, threads) if threads > 1 else (v1, n1, t1)
    return {"value": round(vn, 5), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"median of {nn} GEMVs over the 32 stream matrices (cycled), full "
                      f"14336x4096 each, f64 C oracle, rows split over {threads} threads, {tn:.1f} s",
            "single_core": {"value": round(v1, 5), "cores": 1,
                            "sample": f"median of {n1} stream-matrix GEMVs on one thread, {t1:.1f} s"},
            "host_cpu": host_cpu(), "host_nproc": os.cpu_count()}


def host_cpu() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


PROBE_GRIDS = (256, 384, 512, 768, 1024, 1280, 1536)


def pick_probe_grid(torch, q4, W) -> int:
    """The read probe's workgroup count: the fastest of PROBE_GRIDS over the
    2 GiB buffer (median of 5), so that the measured peak is the probe's
    best, not one grid's (4096 workgroups read about 15% slower)."""
    best = None
    for grid in PROBE_GRIDS:
        q4.read_reduce(W["probe"], grid, partials=W["partials"])
        ts = []
        for _ in range(5):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            q4.read_reduce(W["probe"], grid, partials=W["partials"])
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        t = statistics.median(ts)
        log(f"read_reduce grid {grid}: {wl.PROBE_BYTES / (t * 1e-3) / 1e9:.1f} GB/s")
        if best is None or t < best[0]:
            best = (t, grid)
    return best[1]


def apply_tuned_profile(dev) -> dict | None:
    """Load the device's tuned geometry profile (memory_bandwidth_amd/tuned/)
    into the library, if one exists; returns what was applied."""
    from memory_bandwidth_amd import autotune
    path = autotune.default_profile_path(dev)
    if not os.path.exists(path):
        log("no tuned geometry profile for this device; default plan")
        return None
    n = autotune.apply_profile(path, dev)
    log(f"tuned geometry profile {os.path.basename(path)}: {n} shapes differ from the default plan")
    return {"file": os.path.relpath(path, ROOT), "shapes_set": n}


def run_default(args):
    import torch
    import memory_bandwidth_amd as q4

    dev = torch.device("cuda:0")
    profile = apply_tuned_profile(dev)
    W = setup_stream(torch, q4, dev)
    s = W["shape"]
    g = s.g
    gate(torch, q4, W)
    log("parity gate passed")

    def q4_pass():
        for m, y in zip(W["mats"], W["ys"]):
            q4.gemv_q4(W["x"], m["wq"], m["scales"], m["zeros"], g, out=y)

    def f32_pass():
        for w, y in zip(W["wf"], W["yf"]):
            q4.gemv_f32(W["x"], w, out=y)

    probe_grid = pick_probe_grid(torch, q4, W)

    def probe_pass():
        q4.read_reduce(W["probe"], probe_grid, partials=W["partials"])

    def swiglu_pass():   # gate = matrix 2i, up = matrix 2i + 1
        mats = W["mats"]
        for i in range(wl.STREAM_MATRICES // 2):
            gm, um = mats[2 * i], mats[2 * i + 1]
            q4.gemv_q4_swiglu(W["x"], (gm["wq"], gm["scales"], gm["zeros"]),
                              (um["wq"], um["scales"], um["zeros"]), g, out=W["ys"][i])

    graphs = {"gemv_q4": Graph(q4_pass, torch), "gemv_f32": Graph(f32_pass, torch),
              "read_reduce": Graph(probe_pass, torch), "gemv_q4_swiglu": Graph(swiglu_pass, torch)}
    calls = {"gemv_q4": wl.STREAM_MATRICES, "gemv_f32": wl.STREAM_F32_MATRICES, "read_reduce": 1,
             "gemv_q4_swiglu": wl.STREAM_MATRICES // 2}
    bytes_per_call = {"gemv_q4": wl.q4_weight_bytes(s.N, s.K, s.g),
                      "gemv_f32": wl.f32_weight_bytes(s.N, s.K),
                      "read_reduce": wl.PROBE_BYTES,
                      "gemv_q4_swiglu": 2 * wl.q4_weight_bytes(s.N, s.K, s.g)}

    # ---- two-point / ITERS sweep / ABBA, in the same process, before the
    # timed region (the GPU then runs the timed steps at its steady clocks)
    result = {}
    if not args.quick:
        iters = [int(v) for v in args.iters.split(",")]
        # n counts gemv launches; one 2 GiB read_reduce streams as much as ~70
        # of them, so its sweep uses n / 16 launches.
        scale = {"gemv_q4": 1, "gemv_f32": 1, "read_reduce": 16, "gemv_q4_swiglu": 2}

        def timer(k, n):
            launches = max(1, n // scale[k])
            reps = max(1, launches // calls[k])
            return graphs[k].time(reps) / (reps * calls[k]) * n

        res = sweep(timer, list(graphs), iters, args.runs)
        for k, r in res.items():
            st = summarize(r["samples"])
            gbs = {q: (bytes_per_call[k] / v / 1e9 if v else None) for q, v in st.items() if q != "n"}
            result[k] = {"per_launch_us": {q: (v * 1e6 if isinstance(v, float) else v)
                                           for q, v in st.items()},
                         "GBps_median": gbs["median"], "GBps_best": gbs["min"],
                         "noise_cells": r["noise"], "resolvable_cells": st["n"]}
            log(f"{k:12s} median {gbs['median'] and round(gbs['median'], 1)} GB/s "
                f"(per launch {st['median'] and st['median'] * 1e6:.3f} us; p10-p90 "
                f"{st['p10'] and st['p10'] * 1e6:.3f}-{st['p90'] and st['p90'] * 1e6:.3f}); "
                f"noise cells {r['noise']}")

    # ---- the single-launch read floor at the headline's size
    floor = None if args.quick else run_stream_floor(torch, q4, dev)

    # ---- the contract's timed region: W warm-up steps, then exactly K steps,
    # each step one pass over the 32 matrices.  The K steps are one replay of
    # a graph that holds them (K x 32 launches, captured beforehand), so that
    # no host-side gap between graph launches falls inside the region.
    steps_graph = Graph(lambda: [q4_pass() for _ in range(args.steps)], torch)
    G = graphs["gemv_q4"]
    for _ in range(args.warmup):
        G.g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record()
    steps_graph.g.replay()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    elapsed = start.elapsed_time(end) / 1e3
    del steps_graph
    launches = args.steps * wl.STREAM_MATRICES
    per_launch = elapsed / launches
    value = bytes_per_call["gemv_q4"] / per_launch / 1e9
    log(f"timed region: {args.steps} steps, {launches} launches, {elapsed * 1e3:.3f} ms events, "
        f"{wall * 1e3:.3f} ms wall; {per_launch * 1e6:.3f} us/launch -> {value:.1f} GB/s")

    measured_peak = result.get("read_reduce", {}).get("GBps_median")
    if result.get("read_reduce"):
        result["read_reduce"]["workgroups"] = probe_grid

    traffic = traffic_from_profile(bytes_per_call["gemv_q4"])
    integer = q4.gemv_q4_path(1, s.N, s.K, s.g) == q4.Q4_PATH_INTEGER
    arith = ("x per 32 values as integers of at most 26 bits (seven 4-bit digit planes) plus the exact "
             "fp32 residual of every value more than ~2^12 below the chunk's largest: exact int32 chunk "
             "sums, fp32 residual products, fp32 accumulate; every product within 2^-14 of itself"
             if integer else "(q-z) in fp16, fp32 x, fp32 multiply-add and accumulate")
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i32+f32" if integer else "f32",
        "data": "synthetic",
        "config": {"workload": "stream: 32 distinct int4 g128 matrices, K=4096 N=14336, "
                               "cycled at M=1 (976,224,256 B > L2 + MALL)",
                   "M": 1, "K": 4096, "N": 14336, "group_size": 128,
                   "matrices": wl.STREAM_MATRICES, "bytes_per_call": bytes_per_call["gemv_q4"],
                   "launches_per_step": wl.STREAM_MATRICES,
                   "weights": "int4 codes, fp16 scale + int4 zero per 128, fp32 x and y",
                   "arithmetic": arith, "geometry_profile": profile},
        "roofline": {"bound": "hbm", "achieved": round(value, 2), "peak": SPEC_PEAK_GBS,
                     "unit": "GB/s", "frac": round(value / SPEC_PEAK_GBS, 4),
                     "traffic": traffic},
        "pct_of_spec_peak": round(100 * value / SPEC_PEAK_GBS, 2),
        "measured_peak_GBps": measured_peak and round(measured_peak, 1),
        "pct_of_measured_peak": measured_peak and round(100 * value / measured_peak, 2),
        "two_point": result or None,
        "single_launch_floor_GBps": floor and floor["GBps_median"],
        "pct_of_single_launch_floor": floor and round(100 * value / floor["GBps_median"], 2),
        "cache_class": "hbm-streaming",
    }
    if not args.no_configs:
        line["configs"] = run_configs(torch, q4, dev, W, result, floor,
                                      None if args.no_cpu else args.config_cpu_seconds)
        for c in line["configs"]["cells_cache_resident"] + line["configs"]["cells_hbm_streaming"]:
            if measured_peak and c["GBps_median"]:
                c["frac_of_measured_peak"] = round(c["GBps_median"] / measured_peak, 4)
    if not args.no_blocks:
        line["block_formats"] = run_block_formats(torch, q4, dev)
        line["scan2"] = run_scan(torch, q4, dev)
        line["decoder_layer"] = run_decoder_layer(torch, q4, dev)
        line["ffn_rows"] = run_ffn_rows(torch, q4, W)
    if not args.no_sweep:
        sw = run_bandwidth_sweep(torch, q4, dev, W["probe"])
        ws = wl.STREAM_MATRICES * bytes_per_call["gemv_q4"]
        cl = sw["read_reduce"]["cliffs"]
        lv = cache_level(ws, cl)
        sw["stream_working_set_bytes"] = ws
        line["bandwidth_sweep"] = sw
        # past every cliff of the read sweep: the working set streams from HBM
        line["cache_class"] = ("hbm-streaming" if cl and lv == len(cl)
                               else f"cache-resident: below the read sweep's cliff at {cl[lv]} B")
        line["launch_gap_us"] = round(launch_gap(torch, q4, dev) * 1e6, 3)
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------- the per-config table

L2_BYTES = 32 << 20       # aggregate L2 (4 MB per XCD x 8): the read sweep runs at L2 speed up to here
MALL_BYTES = 256 << 20    # the Infinity Cache: the read sweep's second cliff


def cache_class_of(ws: int) -> str:
    """Where a cell's cycled working set lives, from its size and the read
    sweep's cliffs (64 MiB and 256 MiB on MI355X)."""
    if ws <= L2_BYTES:
        return "cache-resident (L2)"
    if ws <= MALL_BYTES:
        return "cache-resident (Infinity Cache)"
    return "hbm-streaming"


def time_pass(torch, fn, launches: int, reps_target_s: float = 0.02, runs: int = 5) -> dict:
    """Per-launch seconds of a captured pass of `launches` launches, by the
    two-point method over graph replays ((t(2n) - t(n)) / n, n replays of
    about reps_target_s), `runs` kept samples after a warm-up; noise cells
    (t(2n) < 1.2 t(n)) are dropped and counted."""
    G = Graph(fn, torch)
    G.time(2)
    t1 = G.time(1)
    reps = max(1, int(reps_target_s / max(t1, 1e-6)))
    per, noise = [], 0
    while len(per) < runs and noise < 2 * runs:
        a, b = G.time(reps), G.time(2 * reps)
        if resolvable(a, b):
            per.append(two_point(a, b, reps) / launches)
        else:
            noise += 1
    del G
    st = summarize(per)
    st["noise_cells"] = noise
    return st


def cell_record(kernel: str, st: dict, nbytes: int, ws: int, **extra) -> dict:
    """One table cell: per-launch time (median, min, p10-p90), GB/s of the
    algorithmic bytes and its fraction of the 8 TB/s peak, the cache class of
    the cycled working set."""
    med = st["median"]
    rec = {"kernel": kernel, "bytes_per_launch": nbytes, "working_set_bytes": ws,
           "cache_class": cache_class_of(ws),
           "us_per_launch": {q: (round(st[q] * 1e6, 3) if st[q] else None) for q in ("median", "min", "p10", "p90")},
           "runs": st["n"], "noise_cells": st.get("noise_cells", 0),
           "GBps_median": round(nbytes / med / 1e9, 1) if med else None,
           "GBps_best": round(nbytes / st["min"] / 1e9, 1) if st["min"] else None,
           "frac_of_spec": round(nbytes / med / 1e9 / SPEC_PEAK_GBS, 4) if med else None}
    rec.update(extra)
    return rec


def cpu_oracle_cell(problems, budget_s: float, threads: int) -> dict:
    """The oracle, as it stands, on bounded samples of a config: `problems`
    is a list of (x, weights, g, rows) and every call computes the listed
    rows of one problem (rows split into contiguous ranges over `threads`
    host threads); calls cycle through the problems until budget_s of oracle
    time and at least three calls.  GB/s of the rows' int4 bytes, median call."""
    import concurrent.futures
    import numpy as np
    import oracle
    rates, t_used, calls = [], 0.0, 0
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        while t_used < budget_s or calls < 3:
            x, d, g, rows = problems[calls % len(problems)]
            K = x.shape[1]
            nbytes = wl.q4_weight_bytes(len(rows), K, g)
            parts = [r for r in np.array_split(rows, threads) if r.size]
            t0 = time.perf_counter()
            list(ex.map(lambda r: oracle.gemv_q4(x, d["wq"], d["scales"], d["zeros"], g, rows=r), parts))
            dt = time.perf_counter() - t0
            rates.append(nbytes / dt / 1e9)
            t_used += dt
            calls += 1
    return {"GBps": round(statistics.median(rates), 5), "threads": threads, "calls": calls,
            "seconds": round(t_used, 2)}


def cpu_for(problems, budget_s: float) -> dict:
    """cpu_oracle_cell on one thread and on every host thread of one GPU's share."""
    threads = max(1, min(CPU_THREADS_MAX, os.cpu_count() or 1))
    out = {"kind": "oracle", "one_thread": cpu_oracle_cell(problems, budget_s / 2, 1)}
    out["all_threads"] = cpu_oracle_cell(problems, budget_s / 2, threads) if threads > 1 else out["one_thread"]
    out["cores"] = threads
    return out


def dev_mats(torch, dev, host: dict, copies: int, gen) -> list:
    """Matrix 0 from the seeded generator and copies - 1 distinct matrices of
    the same shape on the device: seeded random codes and zero points, every
    scale 2^-7 (the same bytes per call; values do not change the stream)."""
    m0 = {k: torch.from_numpy(v).to(dev) for k, v in host.items()}
    out = [m0]
    for _ in range(copies - 1):
        m = {"wq": torch.randint(0, 256, m0["wq"].shape, dtype=torch.uint8, device=dev, generator=gen),
             "scales": torch.full(m0["scales"].shape, 0x2000, dtype=torch.int16, device=dev),
             "zeros": torch.randint(0, 256, m0["zeros"].shape, dtype=torch.uint8, device=dev, generator=gen)}
        m["scales"] = m["scales"].view(torch.float16)
        out.append(m)
    return out


def run_configs(torch, q4, dev, W, two_pt: dict, floor: dict | None, cpu_s: float) -> dict:
    """The five workloads, each as int4 cells and dense fp32 control cells,
    cache-resident cells (one matrix or one layer looped) apart from
    HBM-streaming ones (distinct copies cycled past the Infinity Cache), each
    with its two-point per-launch statistics, GB/s, fraction of the 8 TB/s
    peak and cache class, and beside it the CPU oracle on bounded samples of
    the same workload (one thread and all threads).  The stream workload's
    cells are the headline's two-point cells and the single-launch read floor."""
    import numpy as np
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.workload_seed(7))
    cells = []

    def add(config, name, rec):
        rec = dict(rec, config=config, name=name)
        cells.append(rec)
        log(f"{config:14s} {name:44s} {rec['kernel']:14s} {rec['us_per_launch']['median']:9.3f} us "
            f"{rec['GBps_median']:8.1f} GB/s  {rec['cache_class']}")

    def q4_pass(x, mats, ys, g, reps=1):
        def fn():
            for _ in range(reps):
                for m, y in zip(mats, ys):
                    q4.gemv_q4(x, m["wq"], m["scales"], m["zeros"], g, out=y)
        return fn

    def f32_pass(x, ws, ys, reps=1):
        def fn():
            for _ in range(reps):
                for w, y in zip(ws, ys):
                    q4.gemv_f32(x, w, out=y)
        return fn

    def dequant(m, g):
        return q4.dequant_q4(m["wq"], m["scales"], m["zeros"], g, want_codes=False)[0]

    cpu = {}
    # ---- one 896 x 896 g32 GEMV
    s = wl.SMALL_896
    d = wl.make_q4_problem(wl.workload_seed(0), s)
    x = torch.from_numpy(d["x"]).to(dev)
    m = {k: torch.from_numpy(v).to(dev) for k, v in d.items() if k != "x"}
    y = [torch.empty((1, s.N), device=dev)]
    nb = wl.q4_weight_bytes(s.N, s.K, s.g)
    add("gemv-896", "single 896x896 g32, one matrix looped", cell_record(
        "gemv_q4", time_pass(torch, q4_pass(x, [m], y, s.g, 64), 64), nb, nb))
    w = dequant(m, s.g)
    add("gemv-896", "single 896x896 fp32 control, one matrix looped", cell_record(
        "gemv_f32", time_pass(torch, f32_pass(x, [w], y, 64), 64), 4 * s.N * s.K, 4 * s.N * s.K))
    cpu_for_ = (lambda probs: cpu_for(probs, cpu_s)) if cpu_s else (lambda probs: None)
    cpu["gemv-896"] = cpu_for_([(d["x"], d, s.g, np.arange(s.N))])
    del m, w

    # ---- the seven decoder-layer GEMVs back to back
    shapes = wl.DECODER_LAYER
    hosts = [wl.make_q4_problem(wl.workload_seed(1), sh, index=i) for i, sh in enumerate(shapes)]
    xs = [torch.from_numpy(h["x"]).to(dev) for h in hosts]
    layer = [{k: torch.from_numpy(v).to(dev) for k, v in h.items() if k != "x"} for h in hosts]
    ys = [torch.empty((1, sh.N), device=dev) for sh in shapes]
    lb = sum(wl.q4_weight_bytes(sh.N, sh.K, sh.g) for sh in shapes)
    fb = sum(4 * sh.N * sh.K for sh in shapes)

    def layer_pass(layers, f32=False, reps=1):
        def fn():
            for _ in range(reps):
                for L in layers:
                    for i, (mm, yy) in enumerate(zip(L, ys)):
                        if f32:
                            q4.gemv_f32(xs[i], mm, out=yy)
                        else:
                            q4.gemv_q4(xs[i], mm["wq"], mm["scales"], mm["zeros"], 32, out=yy)
        return fn

    st = time_pass(torch, layer_pass([layer], reps=16), 16)
    add("decoder-layer", "decoder layer, 7 GEMVs g32, one layer looped", cell_record(
        "gemv_q4 x7", st, lb, lb, unit="per layer"))
    copies = -(-(1 << 30) // lb)
    many = [layer] + [[{k: v.clone() for k, v in mm.items()} for mm in layer] for _ in range(copies - 1)]
    st = time_pass(torch, layer_pass(many), copies)
    add("decoder-layer", f"decoder layer, 7 GEMVs g32, {copies} layers cycled", cell_record(
        "gemv_q4 x7", st, lb, lb * copies, unit="per layer"))
    del many
    fl = [dequant(mm, 32) for mm in layer]
    st = time_pass(torch, layer_pass([fl], f32=True, reps=4), 4)
    add("decoder-layer", "decoder layer, 7 fp32 control GEMVs, one layer looped", cell_record(
        "gemv_f32 x7", st, fb, fb, unit="per layer"))
    fcopies = -(-(1 << 30) // fb)
    fmany = [fl] + [[w.clone() for w in fl] for _ in range(fcopies - 1)]
    st = time_pass(torch, layer_pass(fmany, f32=True), fcopies)
    add("decoder-layer", f"decoder layer, 7 fp32 control GEMVs, {fcopies} layers cycled", cell_record(
        "gemv_f32 x7", st, fb, fb * fcopies, unit="per layer"))
    del fmany, fl, layer
    cpu["decoder-layer"] = cpu_for_([(h["x"], h, 32, np.arange(sh.N)) for h, sh in zip(hosts, shapes)])
    torch.cuda.empty_cache()

    # ---- the LM head 896 -> 151936 g32
    s = wl.LM_HEAD
    d = wl.make_q4_problem(wl.workload_seed(2), s)
    x = torch.from_numpy(d["x"]).to(dev)
    nb = wl.q4_weight_bytes(s.N, s.K, s.g)
    mats = dev_mats(torch, dev, {k: v for k, v in d.items() if k != "x"}, 8, gen)
    y = [torch.empty((1, s.N), device=dev) for _ in mats]
    add("lm-head", "LM head 896->151936 g32, one matrix looped", cell_record(
        "gemv_q4", time_pass(torch, q4_pass(x, mats[:1], y[:1], s.g, 8), 8), nb, nb))
    rot = cell_record("gemv_q4", time_pass(torch, q4_pass(x, mats, y, s.g), 8), nb, 8 * nb)
    del mats
    torch.cuda.empty_cache()
    fl = run_read_floor(torch, q4, dev, nb, 8)
    add("lm-head", "LM head 896->151936 g32, 8 matrices rotated", with_floor(rot, fl))
    add("lm-head", "read_reduce over 8 distinct 78.7 MB buffers (one launch each)",
        cell_record("read_reduce", fl["stats"], nb, 8 * nb, workgroups=fl["workgroups"]))
    mats = dev_mats(torch, dev, {k: v for k, v in d.items() if k != "x"}, 1, gen)
    ws = [dequant(mats[0], s.g)]
    ws.append(ws[0].clone())
    fbytes = 4 * s.N * s.K
    add("lm-head", "LM head fp32 control, 2 matrices rotated", cell_record(
        "gemv_f32", time_pass(torch, f32_pass(x, ws, y[:2]), 2), fbytes, 2 * fbytes))
    del mats, ws
    rng = np.random.default_rng(2)
    cpu["lm-head"] = cpu_for_([(d["x"], d, s.g, np.sort(rng.choice(s.N, 16384, replace=False)))])
    torch.cuda.empty_cache()

    # ---- the 8B-class FFN pair at M = 1, 4, 8
    probs = []
    for M in (1, 4, 8):
        for i, sh in enumerate(wl.ffn_8b(M)):
            h = wl.make_q4_problem(wl.workload_seed(3), sh, index=i)
            xx = torch.from_numpy(h["x"]).to(dev)
            mm = {k: torch.from_numpy(v).to(dev) for k, v in h.items() if k != "x"}
            yy = [torch.empty((M, sh.N), device=dev)]
            nb = wl.q4_weight_bytes(sh.N, sh.K, sh.g)
            path = "integer" if q4.gemv_q4_path(M, sh.N, sh.K, sh.g) == q4.Q4_PATH_INTEGER else "multiply-add"
            st = time_pass(torch, q4_pass(xx, [mm], yy, sh.g, 8), 8)
            flops = 2 * M * sh.N * sh.K
            add("ffn-8b", f"{sh.label}, one matrix looped", cell_record(
                "gemv_q4", st, nb, nb, M=M, path=path,
                TFLOPs=round(flops / st["median"] / 1e12, 2),
                valu_frac_of_fp32_peak=round(flops / st["median"] / FP32_VECTOR_PEAK, 4)))
            if M == 1:
                w = dequant(mm, sh.g)
                add("ffn-8b", f"{sh.label} fp32 control, one matrix looped", cell_record(
                    "gemv_f32", time_pass(torch, f32_pass(xx, [w], yy, 2), 2), 4 * sh.N * sh.K, 4 * sh.N * sh.K))
                del w
            probs.append((h["x"], h, sh.g, np.arange(0, sh.N, max(1, sh.N // 512))))
            del mm
    cpu["ffn-8b"] = cpu_for_(probs)
    torch.cuda.empty_cache()

    # ---- the headline's cells
    s = wl.STREAM_SHAPE
    nb = wl.q4_weight_bytes(s.N, s.K, s.g)
    names = {"gemv_q4": ("stream 4096x14336 g128, 32 matrices cycled", nb, wl.STREAM_MATRICES * nb),
             "gemv_f32": ("stream fp32 control, 4 matrices cycled", 4 * s.N * s.K,
                          wl.STREAM_F32_MATRICES * 4 * s.N * s.K),
             "gemv_q4_swiglu": ("SwiGLU block, 16 gate/up pairs cycled", 2 * nb, wl.STREAM_MATRICES * nb),
             "read_reduce": ("read_reduce over 2 GiB (measured peak)", wl.PROBE_BYTES, wl.PROBE_BYTES)}
    for k, (name, b, ws_) in names.items():
        r = two_pt.get(k)
        if not r:
            continue
        st = {q: (v * 1e-6 if v is not None and q != "n" else v) for q, v in r["per_launch_us"].items()}
        rec = cell_record(k, st, b, ws_)
        if k == "gemv_q4" and floor:
            rec = with_floor(rec, floor)
        if k == "gemv_q4_swiglu":
            fl = run_read_floor(torch, q4, dev, b, wl.STREAM_MATRICES // 2)
            rec = with_floor(rec, fl)
            add("stream", name, rec)
            add("stream", "read_reduce over 16 distinct 61 MB buffers (one launch each)",
                cell_record("read_reduce", fl["stats"], b, ws_, workgroups=fl["workgroups"]))
            continue
        add("stream", name, rec)
    if floor:
        add("stream", "read_reduce over 32 distinct 30.5 MB buffers (one launch each)",
            cell_record("read_reduce", floor["stats"], floor["bytes_per_launch"], floor["working_set_bytes"],
                        workgroups=floor["workgroups"]))
    return {"cells_cache_resident": [c for c in cells if c["cache_class"] != "hbm-streaming"],
            "cells_hbm_streaming": [c for c in cells if c["cache_class"] == "hbm-streaming"],
            "cpu_oracle": {str(k): v for k, v in cpu.items()}}


FLOOR_GRIDS = (256, 512, 768, 1024, 1536, 2048, 4096)


def run_stream_floor(torch, q4, dev) -> dict:
    """The single-launch read floor of the headline's size: read_reduce over
    32 distinct buffers of 30,507,008 B (one stream matrix's bytes; 976 MB
    cycled, past the Infinity Cache), one launch per buffer."""
    nbytes = wl.q4_weight_bytes(wl.STREAM_SHAPE.N, wl.STREAM_SHAPE.K, wl.STREAM_SHAPE.g)
    return run_read_floor(torch, q4, dev, nbytes, wl.STREAM_MATRICES)


def run_read_floor(torch, q4, dev, nbytes: int, count: int) -> dict:
    """The single-launch read floor of a launch that reads nbytes: read_reduce
    over `count` distinct buffers of that size, one launch per buffer,
    non-temporal loads, at the fastest of FLOOR_GRIDS workgroup counts."""
    nf = nbytes // 4
    buf = torch.rand(count * nf, device=dev)
    bufs = [buf[i * nf:(i + 1) * nf] for i in range(count)]
    parts = torch.empty(max(FLOOR_GRIDS), device=dev)
    best = None
    for grid in FLOOR_GRIDS:
        def fn(grid=grid):
            for b in bufs:
                q4.read_reduce(b, grid, partials=parts)
        st = time_pass(torch, fn, len(bufs))
        log(f"single-launch floor over {nbytes} B, {grid} workgroups: {st['median'] * 1e6:.3f} us/launch, "
            f"{nbytes / st['median'] / 1e9:.1f} GB/s")
        if best is None or st["median"] < best[0]["median"]:
            best = (st, grid)
    del buf, bufs
    torch.cuda.empty_cache()
    return {"stats": best[0], "workgroups": best[1], "bytes_per_launch": nbytes,
            "working_set_bytes": count * nbytes,
            "GBps_median": round(nbytes / best[0]["median"] / 1e9, 1)}


def with_floor(rec: dict, fl: dict) -> dict:
    """A streaming cell with the single-launch read floor of its own size."""
    us = fl["stats"]["median"] * 1e6
    return dict(rec, single_launch_floor_us=round(us, 3),
                frac_of_single_launch_floor=round(us / rec["us_per_launch"]["median"], 4))


# ---------------------------------------------------------------- block formats

BLOCK_STREAM_BYTES = 1 << 30    # distinct matrices cycled per shape: at least this many bytes ...
BLOCK_MAX_MATRICES = 64         # ... and at most this many matrices


def block_shapes():
    return [(wl.STREAM_SHAPE.N, wl.STREAM_SHAPE.K, "stream")] + list(wl.BLOCK_SHAPES)


def run_block_formats(torch, q4, dev, reps_target_s: float = 0.02, only=None) -> dict:
    """gemv_block on every format at the stream shape and the cera page's four
    decode shapes.  Matrix 0 of each cell comes from the seeded generator;
    the other distinct matrices (enough to cycle >= 1 GiB, at most 64) are
    seeded random bytes drawn on the device with every binary16 scale field
    set to 2^-7.  Each cell is gated against gemv_f32 on the dequantised
    matrix 0, then timed by two-point differences of graph replays (median
    of three), per launch."""
    out = {}
    seed = wl.workload_seed(5)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    for fmt, (code, e, bb, offs) in wl.BLOCK_FORMATS.items():
        cells = {}
        for N, K, label in block_shapes():
            if only and label not in only:
                continue
            rb = wl.block_row_bytes(fmt, K)
            nbytes = N * rb
            n_mats = max(2, min(BLOCK_MAX_MATRICES, -(-BLOCK_STREAM_BYTES // nbytes)))
            x = torch.from_numpy(wl.make_x(seed, 1, K)).to(dev)
            m0 = torch.from_numpy(wl.make_block_weights(seed, fmt, N, K)).to(dev)
            mats = [m0]
            for _ in range(n_mats - 1):
                m = torch.randint(0, 256, m0.shape, dtype=torch.uint8, device=dev, generator=gen)
                v = m.view(N, K // e, bb)
                for o in offs:
                    v[:, :, o] = 0x00
                    v[:, :, o + 1] = 0x20
                mats.append(m)
            ys = [torch.empty((1, N), dtype=torch.float32, device=dev) for _ in mats]
            w = q4.dequant_block(fmt, m0, K)
            yb = q4.gemv_block(fmt, x, m0)
            yf = q4.gemv_f32(x, w)
            bound = q4.gemv_f32(x.abs(), w.abs())
            err = (yb.double() - yf.double()).abs()
            tol = 2 * (1e-4 * bound.double() + 1e-6)
            if not bool((err <= tol).all()):
                raise SystemExit(f"block parity gate failed: {fmt} {label}: worst err/tol "
                                 f"{float((err / tol).max()):.3g}")
            del w, yf, bound

            def one_pass():
                for mm, y in zip(mats, ys):
                    q4.gemv_block(fmt, x, mm, out=y)

            G = Graph(one_pass, torch)
            G.time(2)
            t1 = G.time(1)
            reps = max(1, int(reps_target_s / max(t1, 1e-6)))
            per = []
            for _ in range(3):
                a, b = G.time(reps), G.time(2 * reps)
                per.append((b - a) / (reps * n_mats))
            t = statistics.median(per)
            gbs = nbytes / t / 1e9
            cells[label] = {"N": N, "K": K, "bytes_per_call": nbytes, "matrices": n_mats,
                            "us_per_launch": round(t * 1e6, 3), "GBps": round(gbs, 1),
                            "frac_of_spec": round(gbs / SPEC_PEAK_GBS, 4),
                            "geometry": list(q4.gemv_block_config(fmt))}
            log(f"block {fmt} {label:12s} N={N} K={K}: {t * 1e6:7.3f} us/launch, {gbs:7.1f} GB/s")
            del mats, ys, G
            torch.cuda.empty_cache()
        out[fmt] = cells
    return out


def run_scan(torch, q4, dev, reps_target_s: float = 0.02) -> dict:
    """scan2 on the Refractometer page's workload, 65,536 vectors x 8 queries
    (D = 768), cycling 64 distinct corpora (805 MB > L2 + MALL): corpus 0
    from the seeded generator, the rest seeded device random words.  Gated
    on 4096 vectors of corpus 0 against the same scores from gemv_f32 (the
    lookup as a GEMV: score[v] = lut[Q, 4D] . onehot(codes[v])), then timed by two-point
    differences of graph replays, per scan."""
    V, Q, D = wl.SCAN_VECTORS, wl.SCAN_QUERIES, wl.SCAN_DIM
    seed = wl.workload_seed(6)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    n_corpora = 64
    c0 = torch.from_numpy(wl.make_scan_codes(seed, V, D).view("int32")).to(dev)
    corpora = [c0] + [torch.randint(-2**31, 2**31 - 1, c0.shape, dtype=torch.int32, device=dev,
                                    generator=gen) for _ in range(n_corpora - 1)]
    lut = torch.from_numpy(wl.make_scan_lut(seed, Q, D)).to(dev)
    outs = [torch.empty((V, Q), dtype=torch.float32, device=dev) for _ in corpora]
    # gate: one-hot expansion of 4096 vectors, scored by the fp32 GEMV
    n = 4096
    sh = torch.arange(16, device=dev, dtype=torch.int64) * 2
    codes = ((c0[:n].to(torch.int64) & 0xFFFFFFFF).unsqueeze(-1) >> sh) & 3          # [n, D/16, 16]
    onehot = torch.nn.functional.one_hot(codes.reshape(n, D), 4).to(torch.float32).reshape(n, 4 * D)
    table = lut.reshape(Q, 4 * D).contiguous()
    ref = q4.gemv_f32(table, onehot).t()               # the table as the 8 activation rows
    bound = q4.gemv_f32(table.abs(), onehot).t()
    got = q4.scan2(c0, lut)[:n]
    err = (got.double() - ref.double()).abs()
    tol = 2 * (1e-4 * bound.double() + 1e-6)
    if not bool((err <= tol).all()):
        raise SystemExit(f"scan parity gate failed: worst err/tol {float((err / tol).max()):.3g}")
    del onehot, codes

    def one_pass():
        for c, o in zip(corpora, outs):
            q4.scan2(c, lut, out=o)

    G = Graph(one_pass, torch)
    G.time(2)
    t1 = G.time(1)
    reps = max(1, int(reps_target_s / max(t1, 1e-6)))
    per = []
    for _ in range(3):
        a, b = G.time(reps), G.time(2 * reps)
        per.append((b - a) / (reps * n_corpora))
    t = statistics.median(per)
    nbytes = V * D // 4
    lds_bytes = V * D * 8 * ((Q + 3) // 4)         # table bytes read from LDS per scan:
                                                   # 16 B per pair of dimensions and query group
    log(f"scan2 {V} x {Q} D={D}: {t * 1e6:.3f} us/scan, {nbytes / t / 1e9:.1f} GB/s of codes, "
        f"{lds_bytes / t / 1e12:.1f} TB/s of LDS table reads")
    res = {"V": V, "Q": Q, "D": D, "bytes_per_call": nbytes, "corpora": n_corpora,
           "us_per_scan": round(t * 1e6, 3), "GBps": round(nbytes / t / 1e9, 1),
           "frac_of_spec": round(nbytes / t / 1e9 / SPEC_PEAK_GBS, 4),
           "lds_table_TBps": round(lds_bytes / t / 1e12, 2),
           "lookups_per_s": round(V * D * Q / t, 1), "config": list(q4.scan2_config())}
    del corpora, outs, G
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- several activation rows

FP32_VECTOR_PEAK = 157.3e12     # MI355X fp32 vector FLOP/s, AMD published
CUS = 256                      # MI355X compute units
SIMDS = CUS * 4                # 4 SIMDs per CU


def run_ffn_rows(torch, q4, W, reps_target_s: float = 0.02) -> dict:
    """The 8B-class FFN pair, 4096 -> 14336 and 14336 -> 4096 at g128, for 1,
    2, 4 and 8 activation rows, cycling the 32 stream matrices (each viewed
    in the shape: the same bytes, 976 MB).  Each cell is gated against
    gemv_f32 on the dequantised matrix 0, then timed by two-point graph
    replays (median of three), per launch, and set against both roofs: HBM
    (weight bytes per call against 8 TB/s) and VALU (2 M N K FLOP per call
    against the fp32 vector peak)."""
    g = wl.STREAM_SHAPE.g
    dev = W["x"].device
    seed = wl.workload_seed(3)
    out = {}
    for label, N, K in (("up 4096->14336", 14336, 4096), ("down 14336->4096", 4096, 14336)):
        G = K // g
        mats = [{"wq": m["wq"].view(N, K // 2), "scales": m["scales"].view(N, G),
                 "zeros": m["zeros"].view(N, (G + 1) // 2)} for m in W["mats"]]
        m0 = mats[0]
        w0 = q4.dequant_q4(m0["wq"], m0["scales"], m0["zeros"], g, want_codes=False)[0]
        nbytes = wl.q4_weight_bytes(N, K, g)
        cells = []
        for M in (1, 2, 4, 8):
            x = torch.from_numpy(wl.make_x(seed, M, K)).to(dev)
            ys = [torch.empty((M, N), dtype=torch.float32, device=dev) for _ in mats]
            y = q4.gemv_q4(x, m0["wq"], m0["scales"], m0["zeros"], g)
            err = (y.double() - q4.gemv_f32(x, w0).double()).abs()
            tol = 2 * (1e-4 * q4.gemv_f32(x.abs(), w0.abs()).double() + 1e-6)
            if not bool((err <= tol).all()):
                raise SystemExit(f"ffn parity gate failed: {label} M={M}: worst err/tol "
                                 f"{float((err / tol).max()):.3g}")

            def one_pass():
                for m, yy in zip(mats, ys):
                    q4.gemv_q4(x, m["wq"], m["scales"], m["zeros"], g, out=yy)

            Gr = Graph(one_pass, torch)
            Gr.time(2)
            t1 = Gr.time(1)
            reps = max(1, int(reps_target_s / max(t1, 1e-6)))
            per = []
            for _ in range(3):
                a, b = Gr.time(reps), Gr.time(2 * reps)
                per.append((b - a) / (reps * len(mats)))
            t = statistics.median(per)
            flops = 2 * M * N * K
            path = "integer" if q4.gemv_q4_path(M, N, K, g) == q4.Q4_PATH_INTEGER else "multiply-add"
            cells.append({"M": M, "path": path, "us_per_launch": round(t * 1e6, 3),
                          "GBps": round(nbytes / t / 1e9, 1),
                          "hbm_frac": round(nbytes / t / 1e9 / SPEC_PEAK_GBS, 4),
                          "TFLOPs": round(flops / t / 1e12, 2),
                          "valu_frac_of_fp32_peak": round(flops / t / FP32_VECTOR_PEAK, 4)})
            log(f"ffn {label} M={M} ({path}): {t * 1e6:7.3f} us/launch, {nbytes / t / 1e9:7.1f} GB/s, "
                f"{flops / t / 1e12:6.2f} TFLOP/s")
            del Gr, ys
        out[label] = {"N": N, "K": K, "group_size": g, "bytes_per_call": nbytes,
                      "matrices": len(mats), "cells": cells}
        del w0
        torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- bandwidth sweep

SWEEP_MIN = 16 << 10            # buffer sizes 16 KiB, 32 KiB, ... 2 GiB
SWEEP_STEPS = 18
SWEEP_GRIDS = (256, 1024, 4096)  # workgroups tried at each size; the best is kept
SWEEP_LAUNCH_BYTES = 1 << 30     # bytes one launch walks: passes = this / size, at most 4096
CLIFF = 0.8                      # the Refractometer page's bandwidth cliff ratio


def find_cliffs(sizes, best, ratio: float = CLIFF):
    """Sizes where the best bandwidth falls below `ratio` of the best at any
    smaller size since the previous cliff (each cliff starts a new level)."""
    cliffs, ref = [], None
    for s, b in zip(sizes, best):
        if ref is not None and b < ratio * ref:
            cliffs.append(s)
            ref = b
        else:
            ref = b if ref is None else max(ref, b)
    return cliffs


def cache_level(nbytes: int, cliffs) -> int:
    """0 for a working set below the first cliff size, 1 below the second, ..."""
    return sum(1 for c in cliffs if nbytes >= c)


def run_bandwidth_sweep(torch, q4, dev, src, samples: int = 25, sample_s: float = 2e-3) -> dict:
    """The Refractometer page's bandwidth sweep: vec4 read-reduce and vec4
    copy over buffers from 16 KiB to 2 GiB, each configuration (workgroup
    count) timed as `samples` samples of back-to-back launches replayed from
    one graph lasting about `sample_s` each (median, p10, p90 per launch);
    the best configuration per size is kept and cliffs are marked by the
    page's 80% rule.  Each launch walks its buffer `passes` times, so that a
    buffer fitting a cache is re-read from it and the cost of a launch is
    spread over about 1 GiB of traffic.  Copy bandwidth counts the bytes read
    and written.  `src` is a float32 device buffer of at least 2 GiB."""
    sizes = [SWEEP_MIN << k for k in range(SWEEP_STEPS)]
    dst = torch.empty(sizes[-1] // 4, dtype=torch.float32, device=dev)
    partials = torch.empty(max(SWEEP_GRIDS), dtype=torch.float32, device=dev)
    out = {"sizes": sizes, "grids": list(SWEEP_GRIDS), "samples": samples}
    for kind in ("read_reduce", "copy"):
        rows = []
        for size in sizes:
            n = size // 4
            passes = max(1, min(4096, SWEEP_LAUNCH_BYTES // size))
            moved = size * passes * (2 if kind == "copy" else 1)
            need = -(-n // 1024)                      # workgroups of 256 lanes x 16 B
            best = None
            for grid in sorted({min(g, need) for g in SWEEP_GRIDS}):
                if kind == "copy":
                    fn = lambda: q4.copy_vec4(src[:n], dst[:n], passes=passes, n_blocks=grid)
                else:
                    fn = lambda: q4.read_reduce_passes(src[:n], grid, passes, partials=partials)
                fn()
                torch.cuda.synchronize()
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                b.synchronize()
                reps = max(1, int(sample_s / max(a.elapsed_time(b) * 1e-3, 1e-7)))
                G = Graph(lambda: [fn() for _ in range(reps)], torch)
                G.time(1)
                per = sorted(G.time(1) / reps for _ in range(samples))
                med = statistics.median(per)
                cell = {"grid": grid, "passes": passes, "GBps_median": moved / med / 1e9,
                        "GBps_p10": moved / per[int(0.9 * (samples - 1))] / 1e9,
                        "GBps_p90": moved / per[int(0.1 * (samples - 1))] / 1e9}
                if best is None or cell["GBps_median"] > best["GBps_median"]:
                    best = cell
                del G
            rows.append({k: (round(v, 1) if isinstance(v, float) else v) for k, v in best.items()})
        gbs = [r["GBps_median"] for r in rows]
        cliffs = find_cliffs(sizes, gbs)
        out[kind] = {"best": rows, "cliffs": cliffs}
        log(f"sweep {kind}: " + ", ".join(f"{s >> 10}K {g:.0f}" for s, g in zip(sizes, gbs)))
        log(f"sweep {kind}: cliffs at " + (", ".join(f"{c >> 10} KiB" for c in cliffs) or "none"))
    del dst
    torch.cuda.empty_cache()
    return out


def launch_gap(torch, q4, dev, launches: int = 256) -> float:
    """Seconds per launch of a kernel that reads nothing and writes one
    float (read_reduce over an empty buffer), back to back in one graph,
    by two-point difference: the fixed cost every launch pays."""
    empty = torch.empty(0, dtype=torch.float32, device=dev)
    part = torch.empty(1, dtype=torch.float32, device=dev)
    G = Graph(lambda: [q4.read_reduce(empty, 1, partials=part) for _ in range(launches)], torch)
    G.time(2)
    per = []
    for _ in range(3):
        a, b = G.time(4), G.time(8)
        per.append((b - a) / (4 * launches))
    return statistics.median(per)


LAYER_COPIES = 64   # distinct decoder layers cycled (64 x 8.6 MB > L2 + MALL)


def run_decoder_layer(torch, q4, dev, reps_target_s: float = 0.02) -> dict:
    """One decoder layer at the gerbil page's MatMul example shapes (WGSL
    Kernel Reference: hidden 896, FFN 4864), with q 896 and k, v 128 wide,
    g32, as seven separate int4 GEMVs
    against four launches: q, k and v stored as one [1152, 896] matrix (their
    rows one after another, one GEMV), o, gate and up fused with the SwiGLU
    combine, down.  Layer 0 comes from the seeded generator, the other
    distinct layers are device copies of it.  The fused q/k/v output is gated
    against gemv_f32 on the dequantised matrix; both passes are timed by
    two-point differences of graph replays (median of three), per layer."""
    seed = wl.workload_seed(1)
    shapes = wl.DECODER_LAYER
    mats = [wl.make_q4_weights(seed, s.N, s.K, s.g, s.s_lo, s.s_hi, index=20 + i)
            for i, s in enumerate(shapes)]
    host = {"sep": mats, "qkv": wl.fuse_rows(*mats[:3])}
    to_dev = lambda m: {k: torch.from_numpy(v).to(dev) for k, v in m.items()}
    l0 = {"sep": [to_dev(m) for m in host["sep"]], "qkv": to_dev(host["qkv"])}
    clone = lambda m: {k: v.clone() for k, v in m.items()}
    layers = [l0] + [{"sep": [clone(m) for m in l0["sep"]], "qkv": clone(l0["qkv"])}
                     for _ in range(LAYER_COPIES - 1)]
    H, F = shapes[0].K, shapes[4].N
    nq = shapes[0].N + shapes[1].N + shapes[2].N
    x = torch.from_numpy(wl.make_x(seed, 1, H, index=20)).to(dev)
    buf = lambda n: torch.empty((1, n), dtype=torch.float32, device=dev)
    ys = [buf(s.N) for s in shapes]
    yqkv, yo, ysw, yd = buf(nq), buf(H), buf(F), buf(H)
    q = l0["qkv"]
    w = q4.dequant_q4(q["wq"], q["scales"], q["zeros"], 32, want_codes=False)[0]
    got = q4.gemv_q4(x, q["wq"], q["scales"], q["zeros"], 32)
    err = (got.double() - q4.gemv_f32(x, w).double()).abs()
    tol = 2 * (1e-4 * q4.gemv_f32(x.abs(), w.abs()).double() + 1e-6)
    if not bool((err <= tol).all()):
        raise SystemExit(f"fused q/k/v gate failed: worst err/tol {float((err / tol).max()):.3g}")
    del w

    def unfused():
        for L in layers:
            for i, (m, y) in enumerate(zip(L["sep"], ys)):
                xin = ys[5] if i == 6 else x          # down reads an FFN-wide activation
                q4.gemv_q4(xin, m["wq"], m["scales"], m["zeros"], 32, out=y)

    def fused():
        for L in layers:
            m, (o, g, u, d) = L["qkv"], L["sep"][3:]
            q4.gemv_q4(x, m["wq"], m["scales"], m["zeros"], 32, out=yqkv)
            q4.gemv_q4(x, o["wq"], o["scales"], o["zeros"], 32, out=yo)
            q4.gemv_q4_swiglu(x, (g["wq"], g["scales"], g["zeros"]),
                              (u["wq"], u["scales"], u["zeros"]), 32, out=ysw)
            q4.gemv_q4(ysw, d["wq"], d["scales"], d["zeros"], 32, out=yd)

    nbytes = sum(wl.q4_weight_bytes(s.N, s.K, s.g) for s in shapes)
    res = {"layer": "hidden 896, ffn 4864, q 896, k/v 128, g32", "bytes_per_layer": nbytes,
           "layers_cycled": LAYER_COPIES}
    for name, fn, launches in (("unfused", unfused, 7), ("fused", fused, 4)):
        G = Graph(fn, torch)
        G.time(2)
        t1 = G.time(1)
        reps = max(1, int(reps_target_s / max(t1, 1e-6)))
        per = []
        for _ in range(3):
            a, b = G.time(reps), G.time(2 * reps)
            per.append((b - a) / (reps * LAYER_COPIES))
        t = statistics.median(per)
        res[name] = {"launches_per_layer": launches, "us_per_layer": round(t * 1e6, 3),
                     "GBps": round(nbytes / t / 1e9, 1)}
        log(f"decoder layer {name:8s} ({launches} launches): {t * 1e6:7.3f} us/layer, "
            f"{nbytes / t / 1e9:7.1f} GB/s of weights")
        del G
    del layers
    torch.cuda.empty_cache()
    return res


def run_blocks_only(args):
    import torch
    import memory_bandwidth_amd as q4
    only = set(args.block_shapes.split(",")) if args.block_shapes else None
    dev = torch.device("cuda:0")
    out = {"unit": "GB/s", "peak": SPEC_PEAK_GBS}
    # the same geometries as the default run
    out["geometry_profile"] = apply_tuned_profile(dev)
    if not only or only - {"scan", "layer", "sweep", "ffn"}:
        out["block_formats"] = run_block_formats(torch, q4, dev, only=only)
    if not only or "scan" in only:
        out["scan2"] = run_scan(torch, q4, dev)
    if not only or "layer" in only:
        out["decoder_layer"] = run_decoder_layer(torch, q4, dev)
    if not only or "ffn" in only:
        out["ffn_rows"] = run_ffn_rows(torch, q4, setup_stream(torch, q4, dev))
        torch.cuda.empty_cache()
    if not only or "sweep" in only:
        src = torch.rand(wl.PROBE_BYTES // 4, device=dev)
        out["bandwidth_sweep"] = run_bandwidth_sweep(torch, q4, dev, src)
        out["launch_gap_us"] = round(launch_gap(torch, q4, dev) * 1e6, 3)
        del src
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------- --pmc-workload

PMC_BLOCK_MATRICES = 8
PMC_READ_KERNEL = "read_reduce_kernel<true>"   # read_reduce's (non-temporal) kernel
PMC_FLOOR_GRID = 2048       # workgroups of the single-launch floor (its fastest in FLOOR_GRIDS)
PMC_FFN_MATRICES = 8        # distinct matrices per FFN projection at M = 4 and 8
PMC_LM_MATRICES = 4         # distinct LM head matrices (315 MB, past the 256 MB MALL)


def run_pmc_workload(args):
    """A short, fixed dispatch sequence for counter collection: 64 gemv_q4 launches
    over the 32 stream matrices, 2 read_reduce and 2 write_fill over 2 GiB (the
    calibration kernels of known size), 4 gemv_f32 launches; the read floor;
    4 and 8 rows of each FFN projection; 8 LM head launches over 4 distinct
    matrices; then 16 gemv_block launches per format at the stream shape over 8
    distinct matrices, and 8 scans of distinct 65,536 x 768 corpora.  The tuned
    geometry profile is applied first, so the counters describe the launches
    the default run times."""
    import torch
    import memory_bandwidth_amd as q4
    dev = torch.device("cuda:0")
    apply_tuned_profile(dev)
    W = setup_stream(torch, q4, dev)
    s = W["shape"]
    for _ in range(2):
        q4.read_reduce(W["probe"], 4096, partials=W["partials"])
        q4.write_fill(W["probe"], 1.0)
    for _ in range(2):
        for m, y in zip(W["mats"], W["ys"]):
            q4.gemv_q4(W["x"], m["wq"], m["scales"], m["zeros"], s.g, out=y)
    for w, y in zip(W["wf"], W["yf"]):
        q4.gemv_f32(W["x"], w, out=y)
    torch.cuda.synchronize()
    del W
    torch.cuda.empty_cache()
    # the single-launch read floor: read_reduce over 32 distinct buffers of one
    # stream matrix's bytes, one launch each
    nf = wl.q4_weight_bytes(s.N, s.K, s.g) // 4
    buf = torch.rand(wl.STREAM_MATRICES * nf, device=dev)
    parts = torch.empty(PMC_FLOOR_GRID, device=dev)
    for i in range(wl.STREAM_MATRICES):
        q4.read_reduce(buf[i * nf:(i + 1) * nf], PMC_FLOOR_GRID, partials=parts)
    torch.cuda.synchronize()
    del buf
    torch.cuda.empty_cache()
    # 4 and 8 activation rows: each FFN projection over distinct matrices
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.workload_seed(3))
    for M in (4, 8):
        for i, sh in enumerate(wl.ffn_8b(M)):
            h = wl.make_q4_problem(wl.workload_seed(3), sh, index=i)
            xx = torch.from_numpy(h["x"]).to(dev)
            mats = dev_mats(torch, dev, {k: v for k, v in h.items() if k != "x"}, PMC_FFN_MATRICES, gen)
            y = torch.empty((M, sh.N), device=dev)
            for m in mats:
                q4.gemv_q4(xx, m["wq"], m["scales"], m["zeros"], sh.g, out=y)
            torch.cuda.synchronize()
            del mats
    torch.cuda.empty_cache()
    # the LM head 896 -> 151936 g32: PMC_LM_MATRICES distinct matrices (more
    # bytes than the MALL holds), each launched twice
    sh = wl.LM_HEAD
    h = wl.make_q4_problem(wl.workload_seed(2), sh)
    xx = torch.from_numpy(h["x"]).to(dev)
    mats = dev_mats(torch, dev, {k: v for k, v in h.items() if k != "x"}, PMC_LM_MATRICES, gen)
    y = torch.empty((1, sh.N), device=dev)
    for _ in range(2):
        for m in mats:
            q4.gemv_q4(xx, m["wq"], m["scales"], m["zeros"], sh.g, out=y)
    torch.cuda.synchronize()
    del mats
    torch.cuda.empty_cache()
    # every block format at the stream shape, 8 distinct matrices launched twice
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.workload_seed(5))
    x = torch.from_numpy(wl.make_x(wl.workload_seed(5), 1, s.K)).to(dev)
    y = torch.empty((1, s.N), dtype=torch.float32, device=dev)
    for fmt, (code, e, bb, offs) in wl.BLOCK_FORMATS.items():
        mats = []
        for _ in range(PMC_BLOCK_MATRICES):
            m = torch.randint(0, 256, (s.N, wl.block_row_bytes(fmt, s.K)), dtype=torch.uint8,
                              device=dev, generator=gen)
            v = m.view(s.N, s.K // e, bb)
            for o in offs:
                v[:, :, o] = 0x00
                v[:, :, o + 1] = 0x20
            mats.append(m)
        for _ in range(2):
            for m in mats:
                q4.gemv_block(fmt, x, m, out=y)
        del mats
    # the scan over 8 distinct corpora of the Refractometer workload
    V, Q, D = wl.SCAN_VECTORS, wl.SCAN_QUERIES, wl.SCAN_DIM
    lut = torch.from_numpy(wl.make_scan_lut(wl.workload_seed(6), Q, D)).to(dev)
    out = torch.empty((V, Q), dtype=torch.float32, device=dev)
    for _ in range(PMC_BLOCK_MATRICES):
        c = torch.randint(-2**31, 2**31 - 1, (V, D // 16), dtype=torch.int32, device=dev, generator=gen)
        q4.scan2(c, lut, out=out)
    torch.cuda.synchronize()
    log("pmc workload done")


# ---------------------------------------------------------------- --summarize

def _rows(pattern):
    out = []
    for f in sorted(glob.glob(pattern, recursive=True)):
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def _kernel_short(name: str) -> str:

    m = re.search(r"(gemv_q4(?:_int|_intm|_fm)?_kernel<[^>]*>|gemv_f32_kernel<[^>]*>|read_reduce_kernel(?:<[^>]*>)?|"
                  r"write_fill_kernel|copy_kernel|dequant_q4_kernel|gemv_blk_kernel<[^>]*>|"
                  r"dequant_blk_kernel<[^>]*>|scan2_kernel<[^>]*>|fm_sum_parts|at::native::\w+|__amd_rocclr_\w+)", name)
    return m.group(1).replace("(anonymous namespace)::", "") if m else name.split("(")[0][:60]


def _kernel_key(r: dict) -> str:
    """Short kernel name, with the grid for read_reduce (whose 2 GiB
    calibration probe and 30.5 MB floor dispatches share one kernel)."""
    k = _kernel_short(r["Kernel_Name"])
    return f"{k} grid {r['Grid_Size']}" if k.startswith("read_reduce") else k


def _keyed_rows(d: str) -> list[tuple[str, dict]]:
    """The counter rows under d, each with its summary key: _kernel_key, and
    " K split" for a multiply-add dispatch that fm_sum_parts follows (the
    down projection with a workspace, whose grid equals the up projection's)."""
    rows = _rows(os.path.join(d, "**", "*counter_collection.csv"))
    kern = {int(r["Dispatch_Id"]): _kernel_key(r) for r in rows}
    ids = sorted(kern)
    split = {a for a, b in zip(ids, ids[1:]) if kern[b] == "fm_sum_parts" and "_fm_" in kern[a]}
    return [(kern[int(r["Dispatch_Id"])] + (" K split" if int(r["Dispatch_Id"]) in split else ""), r)
            for r in rows]


def _probe_key(mean: dict) -> str:
    """The read_reduce dispatch group of the 2 GiB probe: the largest fetch."""
    return max((k for k, c in mean if k.startswith(PMC_READ_KERNEL) and c == "FETCH_SIZE"),
               key=lambda k: mean[(k, "FETCH_SIZE")])


# Counters of the SQ/TA/TCC/GRBM summary, one rocprofv3 --pmc pass each
# (per-block limits: 8 SQ, 4 TCC, 2 TA, 2 GRBM per pass).
PMC_COUNTER_PASSES = (
    "SQ_WAVES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY "
    "SQ_INSTS_LDS SQ_INSTS_VMEM_RD",
    "TA_BUSY_avr TA_BUFFER_READ_WAVEFRONTS_sum TCC_REQ_sum TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE "
    "GRBM_COUNT",
    "SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS SQ_INSTS_VALU_FMA_F32 "
    "SQ_INSTS_VALU_INT32 SQ_INSTS_VALU_ADD_F32 SQ_INSTS_VALU_MUL_F32",
)
CLOCK_GHZ = 2.4            # MI355X peak engine clock, for cycle counts over a dispatch


def summarize_counters(dirs: list[str], name: str, command: str) -> str:
    """rocprofv3 --pmc runs of --pmc-workload, one per PMC_COUNTER_PASSES entry
    -> profiles/<name>.md: per kernel (and grid, for read_reduce), the mean
    of every counter per dispatch, the mean dispatch duration under the
    profiler, and the VALU issue figures derived from them."""
    per, dur, grid = {}, {}, {}
    for d in dirs:
        for k, r in _keyed_rows(d):
            if not re.match(r"(gemv_q4|gemv_blk|read_reduce|fm_sum_parts|scan2)", k):
                continue
            per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            dur.setdefault(k, {})[(d, r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
            grid[k] = int(r["Grid_Size"]) // int(r["Workgroup_Size"])
    lines = [f"# {name}: rocprofv3 counters per dispatch", "", f"command: `{command}`", "",
             "Means over the dispatches of each kernel in one --pmc-workload run per pass "
             "(the stream kernel: 64 launches over 32 matrices; the read floor: 32 buffers of "
             "30.5 MB, one launch each; 4 and 8 rows: 8 matrices per FFN projection, the "
             "up projection 4096 -> 14336 plain, the down projection 14336 -> 4096 split over "
             "K with a workspace (marked K split, then fm_sum_parts adds the parts); the LM "
             "head 896 -> 151936 g32 (the short-row kernel, 32 lanes per row): 8 launches over "
             "4 matrices; the block formats at the stream shape: 16 launches over 8 matrices "
             "each).  "
             "Durations are those of the counter runs (serialised dispatches).", ""]
    ctrs = [c for p in PMC_COUNTER_PASSES for c in p.split()]
    for k in sorted(per):
        c = {n: statistics.mean(v) for n, v in per[k].items()}
        us = statistics.mean(dur[k].values()) / 1e3
        lines += [f"## {k} ({grid[k]} workgroups)", "", "| counter | mean per dispatch |", "|---|---|"]
        lines += [f"| {n} | {c[n]:.1f} |" for n in ctrs if n in c]
        lines += ["", f"mean dispatch duration under the profiler: {us:.2f} us."]
        if "SQ_INSTS_VALU" in c and "SQ_WAVES" in c and c["SQ_WAVES"]:
            rate = c["SQ_INSTS_VALU"] / (SIMDS * us * 1e3)
            lines.append(f"VALU: {c['SQ_INSTS_VALU'] / c['SQ_WAVES']:.0f} wavefront-instructions per "
                         f"wavefront; {rate:.3f} issued per SIMD per ns over the dispatch "
                         f"({SIMDS} SIMDs; one SIMD issues at most about 0.95 per ns with two or "
                         "more wavefronts ready, 0.5 with one).")
        if "SQ_ACTIVE_INST_VALU" in c and "SQ_INSTS_VALU" in c and c["SQ_INSTS_VALU"]:
            lines.append(f"SQ_ACTIVE_INST_VALU / SQ_INSTS_VALU = "
                         f"{c['SQ_ACTIVE_INST_VALU'] / c['SQ_INSTS_VALU']:.2f}.")
        if "SQ_WAIT_INST_ANY" in c and "SQ_ACTIVE_INST_ANY" in c and c["SQ_ACTIVE_INST_ANY"]:
            lines.append(f"SQ_WAIT_INST_ANY / SQ_ACTIVE_INST_ANY = "
                         f"{c['SQ_WAIT_INST_ANY'] / c['SQ_ACTIVE_INST_ANY']:.2f}.")
        if "GRBM_GUI_ACTIVE" in c:
            lines.append(f"GRBM_GUI_ACTIVE {c['GRBM_GUI_ACTIVE']:.0f} cycles per dispatch.")
        if "SQ_LDS_IDX_ACTIVE" in c:
            cyc = CUS * us * 1e3 * CLOCK_GHZ
            lines.append(f"LDS busy {100 * c['SQ_LDS_IDX_ACTIVE'] / cyc:.1f}% of the dispatch's CU cycles "
                         f"({CUS} CUs at {CLOCK_GHZ} GHz); bank-conflict cycles "
                         f"{c.get('SQ_LDS_BANK_CONFLICT', 0):.0f}.")
        if "SQ_INSTS_VALU_FMA_F32" in c and c.get("SQ_INSTS_VALU"):
            lines.append(f"fp32 FMA {100 * c['SQ_INSTS_VALU_FMA_F32'] / c['SQ_INSTS_VALU']:.1f}% of the VALU "
                         "instructions.")
        lines.append("")
    out = os.path.join(PROFILES, name + ".md")
    open(out, "w").write("\n".join(lines) + "\n")
    return out


def summarize_stats(d: str, name: str, command: str) -> str:
    """rocprofv3 --kernel-trace --stats CSV under d -> profiles/<name>.md."""
    stats = _rows(os.path.join(d, "**", "*kernel_stats.csv"))
    lines = [f"# {name}: rocprofv3 kernel statistics", "", f"command: `{command}`", "",
             "| kernel | calls | avg ns | min ns | max ns | % of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r.get("Percentage", 0) or 0)):
        lines.append(f"| {_kernel_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                     f"{float(r['MinNs']):.0f} | {float(r['MaxNs']):.0f} | "
                     f"{float(r['Percentage']):.2f} |")
    # per-kernel bandwidth lines for the workload the summary is named for
    q = [r for r in stats if re.search(r"gemv_q4(_int)?_kernel<8, 64, 2, 4, 1, false, false", r["Name"])]
    if q and name.startswith("gemv_q4_stream"):
        avg = float(q[0]["AverageNs"]) * 1e-9
        b = wl.q4_weight_bytes(wl.STREAM_SHAPE.N, wl.STREAM_SHAPE.K, wl.STREAM_SHAPE.g)
        lines += ["", f"gemv_q4 average kernel duration {avg * 1e6:.3f} us -> "
                      f"{b / avg / 1e9:.1f} GB/s of algorithmic bytes ({b} B per launch)."]
    sc = [r for r in stats if "scan2_kernel" in r["Name"]]
    if sc and name.startswith("scan2"):
        V, D = wl.SCAN_VECTORS, wl.SCAN_DIM
        avg = float(sc[0]["AverageNs"]) * 1e-9
        lines += ["", f"scan2 ({V} vectors x {wl.SCAN_QUERIES} queries, D = {D}): average "
                      f"{avg * 1e6:.3f} us -> {V * D / 4 / avg / 1e9:.1f} GB/s of codes "
                      f"({V * D // 4} B per scan), {V * D * 16 / avg / 1e12:.1f} TB/s of LDS "
                      "table reads (16 B per vector and pair of dimensions, for each group of "
                      "four queries)."]
    blk = [r for r in stats if "gemv_blk_kernel" in r["Name"]]
    if blk and name.startswith("gemv_block_stream"):
        s = wl.STREAM_SHAPE
        lines += ["", f"gemv_block at the stream shape (N={s.N}, K={s.K}; each kernel above ran "
                      "only that shape):"]
        for r in blk:
            fmt = re.search(r"FmtQ(\w+?),", r["Name"]).group(1).lower()
            b = wl.block_row_bytes("q" + fmt, s.K) * s.N
            avg = float(r["AverageNs"]) * 1e-9
            lines.append(f"- q{fmt}: average {avg * 1e6:.3f} us -> {b / avg / 1e9:.1f} GB/s "
                         f"({b} B per launch)")
    out = os.path.join(PROFILES, name + ".md")
    open(out, "w").write("\n".join(lines) + "\n")
    return out


def summarize_pmc(fetch_dir: str, write_dir: str, name: str, command: str) -> str:
    """Two rocprofv3 --pmc runs of --pmc-workload (FETCH_SIZE, then WRITE_SIZE,
    KiB per dispatch) -> profiles/<name>.md and the JSON bench.py reads for
    roofline.traffic.  Each counter is scaled by what it reads for a probe of
    known size: read_reduce streams PROBE_BYTES, write_fill writes PROBE_BYTES."""
    per = {}
    for d, ctr in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        for k, r in _keyed_rows(d):
            if r["Counter_Name"] == ctr:
                per.setdefault((k, ctr), []).append(float(r["Counter_Value"]))
    mean = {k: statistics.mean(v) for k, v in per.items()}
    probe = _probe_key(mean)
    fetch_factor = wl.PROBE_BYTES / (mean[(probe, "FETCH_SIZE")] * 1024)
    write_factor = wl.PROBE_BYTES / (mean[("write_fill_kernel", "WRITE_SIZE")] * 1024)
    # the stream kernel: the gemv_q4 kernel with the most dispatches (2 x 32)
    # (the multiply-add launches at 4 and 8 rows: 8 per FFN projection)
    qk = max((k for k, c in mean if k.startswith("gemv_q4_") and c == "FETCH_SIZE"),
             key=lambda k: len(per[(k, "FETCH_SIZE")]))
    s = wl.STREAM_SHAPE
    alg = wl.q4_weight_bytes(s.N, s.K, s.g)
    fetch_b = mean[(qk, "FETCH_SIZE")] * 1024 * fetch_factor
    write_b = mean[(qk, "WRITE_SIZE")] * 1024 * write_factor
    summary = {"kernel": qk, "workload": "stream 4096x14336 g128, M=1, 32 distinct matrices",
               "kernel_source_sha256_16": kernel_source_hash(),
               "fetch_factor": round(fetch_factor, 5), "write_factor": round(write_factor, 5),
               "gemv_q4_fetch_bytes_per_launch": round(fetch_b),
               "gemv_q4_write_bytes_per_launch": round(write_b),
               "gemv_q4_hbm_bytes_per_launch": round(fetch_b + write_b),
               "algorithmic_bytes_per_launch": alg,
               "x_and_y_bytes_per_launch": 4 * s.K + 4 * s.N,
               "command": command}
    json.dump(summary, open(PMC_SUMMARY, "w"), indent=1)
    lines = [f"# {name}: HBM traffic from rocprofv3 counters", "", f"command: `{command}`", "",
             f"Calibration: read_reduce over {wl.PROBE_BYTES} B reads FETCH_SIZE "
             f"{mean[(probe, 'FETCH_SIZE')]:.1f} KiB -> factor {fetch_factor:.4f}; "
             f"write_fill over {wl.PROBE_BYTES} B reads WRITE_SIZE "
             f"{mean[('write_fill_kernel', 'WRITE_SIZE')]:.1f} KiB -> factor {write_factor:.4f}.", "",
             "| kernel | counter | dispatches | mean KiB/dispatch | scaled bytes/dispatch |",
             "|---|---|---|---|---|"]
    for (k, ctr), v in sorted(per.items()):
        f = fetch_factor if ctr == "FETCH_SIZE" else write_factor
        lines.append(f"| {k} | {ctr} | {len(v)} | {statistics.mean(v):.1f} | "
                     f"{statistics.mean(v) * 1024 * f:.0f} |")
    lines += ["", f"gemv_q4 per launch: {fetch_b + write_b:.0f} B of HBM traffic against "
                  f"{alg} algorithmic bytes (+{4 * s.K + 4 * s.N} B of x and y): ratio "
                  f"{(fetch_b + write_b) / alg:.4f}.",
              f"Kernel source sha256[:16] {summary['kernel_source_sha256_16']}."]
    for k, _ in sorted(mean):
        if _ != "FETCH_SIZE":
            continue
        m = re.search(r"gemv_blk_kernel<FmtQ(\w+?),", k)
        if m:
            fmt = "q" + m.group(1).lower()
            a = wl.block_row_bytes(fmt, s.K) * s.N
            f = mean[(k, "FETCH_SIZE")] * 1024 * fetch_factor
            lines.append(f"gemv_block {fmt} per launch (stream shape): {f:.0f} B fetched against "
                         f"{a} algorithmic bytes: ratio {f / a:.4f}.")
        elif k.startswith("gemv_q4_fm_kernel"):
            a = wl.q4_weight_bytes(s.N, s.K, s.g)
            f = mean[(k, "FETCH_SIZE")] * 1024 * fetch_factor
            w = mean.get((k, "WRITE_SIZE"), 0.0) * 1024 * write_factor
            lines.append(f"{k} per launch (an FFN projection, {a} B of weights): {f:.0f} B fetched "
                         f"(ratio {f / a:.4f}), {w:.0f} B written.")
        elif k.startswith("gemv_q4_int_kernel<8, 32,"):
            lm = wl.LM_HEAD
            a = wl.q4_weight_bytes(lm.N, lm.K, lm.g)
            f = mean[(k, "FETCH_SIZE")] * 1024 * fetch_factor
            lines.append(f"{k} per launch (the LM head 896 -> 151936 g32, {a} B): {f:.0f} B "
                         f"fetched, ratio {f / a:.4f}.")
        elif k == "fm_sum_parts":
            f = mean[(k, "FETCH_SIZE")] * 1024 * fetch_factor
            w = mean.get((k, "WRITE_SIZE"), 0.0) * 1024 * write_factor
            lines.append(f"fm_sum_parts per launch (the K parts of a split down projection): "
                         f"{f:.0f} B fetched, {w:.0f} B written.")
        elif k.startswith("scan2_kernel"):
            a = wl.SCAN_VECTORS * wl.SCAN_DIM // 4
            f = mean[(k, "FETCH_SIZE")] * 1024 * fetch_factor
            lines.append(f"scan2 per launch (65,536 x 768 codes, 8 queries): {f:.0f} B fetched "
                         f"against {a} B of codes: ratio {f / a:.4f} (each code is read by two "
                         "workgroups, one per group of four queries, on one XCD: the second "
                         "read is served by its L2).")
    out = os.path.join(PROFILES, name + ".md")
    open(out, "w").write("\n".join(lines) + "\n")
    return out


def summarize_profile(args):
    os.makedirs(PROFILES, exist_ok=True)
    if args.summarize_counters:
        log("wrote", summarize_counters([args.summarize] + args.summarize_counters, args.name, args.command))
    elif args.summarize_write:
        log("wrote", summarize_pmc(args.summarize, args.summarize_write, args.name, args.command))
    else:
        log("wrote", summarize_stats(args.summarize, args.name, args.command))


# ---------------------------------------------------------------- main

def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--iters", default="64,256,1024", help="ITERS sweep, in launches")
    ap.add_argument("--runs", type=int, default=3, help="kept runs per cell (>= 3)")
    ap.add_argument("--quick", action="store_true", help="skip the two-point sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-blocks", action="store_true", help="skip the block-format cells")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config table")
    ap.add_argument("--config-cpu-seconds", type=float, default=3.0,
                    help="CPU oracle seconds per config of the table (half on one thread, half on all)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the 16 KiB - 2 GiB bandwidth sweep")
    ap.add_argument("--blocks-only", action="store_true", help="only the block-format cells")
    ap.add_argument("--block-shapes", default="",
                    help="with --blocks-only: comma list of shape labels (stream, 'lm head', ..., scan, layer, ffn, sweep)")
    ap.add_argument("--pmc-workload", action="store_true")
    ap.add_argument("--summarize", metavar="DIR", help="rocprofv3 CSV dir (stats, or FETCH_SIZE pmc)")
    ap.add_argument("--summarize-write", metavar="DIR", help="WRITE_SIZE pmc dir (with --summarize)")
    ap.add_argument("--summarize-counters", metavar="DIR", nargs="+",
                    help="further pmc dirs (with --summarize): the SQ/TA/TCC/GRBM counter summary")
    ap.add_argument("--name", default="summary")
    ap.add_argument("--command", default="")
    args = ap.parse_args(argv)
    if args.summarize:
        return summarize_profile(args)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the int4 GEMV shards by output rows; the benchmark measures one GPU)", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0 or args.runs < 1:
        print("--steps must be >= 1, --warmup >= 0, --runs >= 1", file=sys.stderr)
        return 2
    if args.pmc_workload:
        return run_pmc_workload(args)
    if args.blocks_only:
        return run_blocks_only(args)
    return run_default(args)


if __name__ == "__main__":
    sys.exit(main() or 0)
