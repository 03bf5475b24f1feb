"""Geometry autotuner and per-device profile for gemv_q4.

Follows the method of Refractometer ("What each sweep measures", q4 GEMV,
and its timing paragraph): sweep the GEMV's geometry knobs at the real
shapes, check every configuration against a reference before it is timed so
that a fast kernel with wrong output cannot win, time each with a median and
p10-p90 over 25 samples of about 2 ms after warm-up, mark configurations
that fall below 75% of the best as cliffs, and keep the winners as a JSON
profile keyed by the device.

Knobs: the arithmetic path (multiply-add or integer), wavefronts per
workgroup and the K-split, i.e. every combination gemv_q4_set_geometry
accepts for the shape; the library plans the rest (rows per workgroup,
chunk positions per lane, x segments).  Candidates are timed through
gemv_q4 without a workspace, the plan the knobs set: where gemv_q4_ws splits
K over workgroups its plan takes the wavefront split from the rows, not from
the knob.

Reference: the library's dense fp32 GEMV on the device-dequantised weights,
with the bound |x| . |W|^T from the same GEMV of absolute values; a
candidate must agree within 2 (1e-4 bound + 1e-6).  Inputs are random and
generated on the device: codes and zero points uniform, scales uniform in
[0.002, 0.02], x ~ N(0, 1).

The same method covers the other kernels whose knobs the pages sweep: the
block-format GEMV (row slots per lane, wavefronts per workgroup, workgroups
per CU, per format, at the stream shape and the cera page's decode shapes;
reference: gemv_f32 on dequant_block's weights) and the 2-bit scan (table in
LDS or memory, vectors per thread, workgroup size, threads per vector, at
the Refractometer page's 65,536 x 8 workload with D = 768; reference:
gemv_f32 on the one-hot expansion of 4096 vectors).  Their settings are
process-wide, one per format and one for the scan, so a winner is applied
only where it holds: a block format's at both large shapes (the stream and
the 65,536-row LM head), the scan's at its workload, and in both cases only
if it beats the library's default by at least 3%.

    python -m memory_bandwidth_amd.autotune [--out FILE] [--quick] [--only q4,blocks,scan]

writes the profile (default: tuned/<device>.json beside this file);
apply_profile() loads the one for the current device into the library.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import torch

import memory_bandwidth_amd as q4

TUNED_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tuned")
SAMPLES = 25
SAMPLE_S = 2e-3
CLIFF = 0.75
STREAM_BYTES = 1 << 30          # matrices cycled per sample: at least this many bytes ...
MAX_MATRICES = 64               # ... but no more than this many distinct matrices

# The shapes the library is used at: (M, N, K, group_size).
SHAPES = [
    (1, 896, 896, 32), (1, 128, 896, 32), (1, 4864, 896, 32), (1, 896, 4864, 32),
    (1, 151936, 896, 32),
    (1, 14336, 4096, 128), (1, 4096, 14336, 128),
    (4, 14336, 4096, 128), (4, 4096, 14336, 128),
    (8, 14336, 4096, 128), (8, 4096, 14336, 128),
]


def device_key(dev: torch.device | None = None) -> str:
    p = torch.cuda.get_device_properties(dev or torch.device("cuda:0"))
    return f"{p.gcnArchName.split(':')[0]}-{p.multi_processor_count}cu"


def default_profile_path(dev: torch.device | None = None) -> str:
    return os.path.join(TUNED_DIR, device_key(dev) + ".json")


def q4_bytes(N: int, K: int, g: int) -> int:
    G = K // g
    return N * K // 2 + 2 * N * G + N * ((G + 1) // 2)


def _random_matrix(N: int, K: int, g: int, gen: torch.Generator, dev: torch.device) -> dict:
    G = K // g
    wq = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=dev, generator=gen)
    zeros = torch.randint(0, 256, (N, (G + 1) // 2), dtype=torch.uint8, device=dev, generator=gen)
    scales = (torch.rand((N, G), device=dev, generator=gen) * 0.018 + 0.002).to(torch.float16)
    return {"wq": wq, "scales": scales, "zeros": zeros}


def candidates(M: int, N: int, K: int, g: int) -> list[dict]:
    """Every distinct geometry gemv_q4_set_geometry accepts for the shape."""
    seen, out = set(), []
    for path in (q4.Q4_PATH_FMA, q4.Q4_PATH_INTEGER):
        for waves in (0, 4, 8, 16):
            for ksplit in (0, 1, 2, 4):
                try:
                    q4.gemv_q4_set_geometry(M, N, K, g, path, waves, ksplit)
                except q4.Q4Error:
                    continue
                geo = q4.gemv_q4_geometry(M, N, K, g)
                key = (path, tuple(sorted(geo.items())))
                if key not in seen:
                    seen.add(key)
                    out.append({"path": path, "waves": geo["block"] // 64,
                                "ksplit": geo["ksplit"], "geometry": geo})
    q4.gemv_q4_clear_geometry()
    return out


class _Case:
    """Inputs of one shape, resident on the device, and its reference."""

    def __init__(self, M: int, N: int, K: int, g: int, dev: torch.device, seed: int):
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        nb = q4_bytes(N, K, g)
        self.n_mats = max(1, min(MAX_MATRICES, -(-STREAM_BYTES // nb)))
        self.x = torch.randn((M, K), device=dev, generator=gen)
        self.mats = [_random_matrix(N, K, g, gen, dev) for _ in range(self.n_mats)]
        self.ys = [torch.empty((M, N), device=dev) for _ in self.mats]
        m0 = self.mats[0]
        w = q4.dequant_q4(m0["wq"], m0["scales"], m0["zeros"], g, want_codes=False)[0]
        self.ref = q4.gemv_f32(self.x, w).double()
        self.tol = 2 * (1e-4 * q4.gemv_f32(self.x.abs(), w.abs()).double() + 1e-6)
        del w
        self.shape = (M, N, K, g)
        self.bytes = nb

    def check(self) -> bool:
        M, N, K, g = self.shape
        m0 = self.mats[0]
        y = q4.gemv_q4(self.x, m0["wq"], m0["scales"], m0["zeros"], g, workspace=False).double()
        return bool(((y - self.ref).abs() <= self.tol).all())

    def time(self) -> dict:
        M, N, K, g = self.shape

        def one_pass():
            for m, y in zip(self.mats, self.ys):
                q4.gemv_q4(self.x, m["wq"], m["scales"], m["zeros"], g, out=y, workspace=False)

        return _sample(one_pass, self.n_mats, self.bytes)


def _sample(one_pass, calls: int, nbytes: int) -> dict:
    """Median and p10-p90 per call over SAMPLES replays of about SAMPLE_S
    each; one_pass makes `calls` calls of `nbytes` algorithmic bytes each."""
    one_pass()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    one_pass()
    torch.cuda.synchronize()
    per_pass = max(time.perf_counter() - t0, 1e-6)
    passes = max(1, min(64, round(SAMPLE_S / per_pass)))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(passes):
            one_pass()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    samples = []
    for _ in range(SAMPLES):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        b.synchronize()
        samples.append(a.elapsed_time(b) * 1e-3 / (passes * calls))
    samples.sort()
    med = statistics.median(samples)
    return {"median_us": med * 1e6, "p10_us": samples[int(0.1 * (SAMPLES - 1))] * 1e6,
            "p90_us": samples[int(0.9 * (SAMPLES - 1))] * 1e6, "GBps": nbytes / med / 1e9}


def _rank(results: list[dict]) -> dict:
    """The fastest candidate that passed parity; flags every timed one that
    falls below CLIFF of it."""
    timed = [r for r in results if r["parity"]]
    if not timed:
        raise RuntimeError("no configuration passed the parity check")
    best = min(timed, key=lambda r: r["median_us"])
    for r in timed:
        r["frac_of_best"] = best["median_us"] / r["median_us"]
        r["cliff"] = r["frac_of_best"] < CLIFF
    return best


def tune_shape(M: int, N: int, K: int, g: int, dev: torch.device, seed: int = 1) -> dict:
    case = _Case(M, N, K, g, dev, seed)
    default = {"path": q4.gemv_q4_path(M, N, K, g), **q4.gemv_q4_geometry(M, N, K, g)}
    results = []
    for cand in candidates(M, N, K, g):
        q4.gemv_q4_set_geometry(M, N, K, g, cand["path"], cand["waves"], cand["ksplit"])
        ok = case.check()
        entry = dict(cand, parity=ok)
        if ok:
            entry.update(case.time())
        entry["default"] = (cand["path"] == default["path"] and
                            all(cand["geometry"][k] == default[k] for k in cand["geometry"]))
        results.append(entry)
        q4.gemv_q4_clear_geometry()
    best = _rank(results)
    n_mats = case.n_mats
    del case
    torch.cuda.empty_cache()
    return {"M": M, "N": N, "K": K, "group_size": g, "matrices_cycled": n_mats,
            "best": {k: best[k] for k in ("path", "waves", "ksplit", "median_us", "p10_us",
                                          "p90_us", "GBps", "default")},
            "candidates": results}


# ---------------------------------------------------------------- block formats and scan

# (N, K): the stream shape, the cera page's LM head, FFN gate/up, FFN down, attention.
BLOCK_SHAPES = [(14336, 4096), (65536, 1024), (2816, 1024), (1024, 2816), (1024, 1024)]
BLOCK_LARGE = BLOCK_SHAPES[:2]
# Byte offsets, within a block, of the binary16 fields that scale it (d, and
# dmin for Q4_K / Q5_K): random matrices set them to 2^-7 so that no weight
# is infinite or NaN.
SCALE_FIELDS = {"q4_0": (0,), "q8_0": (0,), "q4_k": (0, 2), "q5_k": (0, 2), "q6_k": (208,)}
APPLY_GAIN = 1.03               # a process-wide winner must beat the default by this much
SCAN_WORKLOAD = (65536, 8, 768)  # vectors, queries, dimensions


def block_candidates(fmt) -> list[tuple[int, int, int]]:
    """(rows per lane, wavefronts, workgroups per CU) settings the library
    accepts for the format; (0, 0, 0) is its own default plan."""
    out = [(0, 0, 0)]
    for r in (1, 2, 4):
        for w in (4, 8):
            for gpc in (0, 1, 2, 4):
                try:
                    q4.gemv_block_set_config(fmt, r, w, gpc)
                except q4.Q4Error:
                    continue
                out.append((r, w, gpc))
    q4.gemv_block_set_config(fmt, 0, 0, 0)
    return out


def tune_block(fmt, N: int, K: int, dev: torch.device, seed: int = 2) -> dict:
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    elems, bb = q4.block_geometry(fmt)
    nbytes = N * (K // elems) * bb
    n_mats = max(2, min(MAX_MATRICES, -(-STREAM_BYTES // nbytes)))
    mats = []
    for _ in range(n_mats):
        m = torch.randint(0, 256, (N, K // elems * bb), dtype=torch.uint8, device=dev, generator=gen)
        v = m.view(N, K // elems, bb)
        for o in SCALE_FIELDS[fmt]:
            v[:, :, o] = 0x00
            v[:, :, o + 1] = 0x20
        mats.append(m)
    x = torch.randn((1, K), device=dev, generator=gen)
    ys = [torch.empty((1, N), device=dev) for _ in mats]
    w = q4.dequant_block(fmt, mats[0], K)
    ref = q4.gemv_f32(x, w).double()
    tol = 2 * (1e-4 * q4.gemv_f32(x.abs(), w.abs()).double() + 1e-6)
    del w

    def one_pass():
        for m, y in zip(mats, ys):
            q4.gemv_block(fmt, x, m, out=y)

    results = []
    try:
        for cfg in block_candidates(fmt):
            q4.gemv_block_set_config(fmt, *cfg)
            y = q4.gemv_block(fmt, x, mats[0]).double()
            entry = {"config": list(cfg), "parity": bool(((y - ref).abs() <= tol).all())}
            if entry["parity"]:
                entry.update(_sample(one_pass, n_mats, nbytes))
            results.append(entry)
    finally:
        q4.gemv_block_set_config(fmt, 0, 0, 0)
    best = _rank(results)
    del mats, ys
    torch.cuda.empty_cache()
    default = next(r for r in results if r["config"] == [0, 0, 0])
    return {"format": fmt, "N": N, "K": K, "matrices_cycled": n_mats,
            "best": {"config": best["config"], "median_us": best["median_us"], "GBps": best["GBps"],
                     "default_us": default.get("median_us")},
            "candidates": results}


def scan_candidates() -> list[tuple[int, int, int, int]]:
    """(table in LDS, vectors per thread, workgroup size, threads per vector);
    (0, 0, 0, 0) is the library's default; the table read from memory is
    tried in the page's own tail shape only (it is about ten times slower)."""
    out = [(0, 0, 0, 0), (0, 1, 256, 1)]
    for vpt in (1, 2):
        for tpg in (64, 256, 1024):
            for tpv in (1, 2, 4, 8):
                out.append((1, vpt, tpg, tpv))
    return out


def tune_scan(dev: torch.device, seed: int = 3) -> dict:
    V, Q, D = SCAN_WORKLOAD
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    n_corpora = 64
    corpora = [torch.randint(-2**31, 2**31 - 1, (V, D // 16), dtype=torch.int32, device=dev,
                             generator=gen) for _ in range(n_corpora)]
    lut = torch.randn((Q, D, 4), device=dev, generator=gen)
    outs = [torch.empty((V, Q), device=dev) for _ in corpora]
    n = 4096
    sh = torch.arange(16, device=dev, dtype=torch.int64) * 2
    codes = ((corpora[0][:n].to(torch.int64) & 0xFFFFFFFF).unsqueeze(-1) >> sh) & 3
    onehot = torch.nn.functional.one_hot(codes.reshape(n, D), 4).to(torch.float32).reshape(n, 4 * D)
    table = lut.reshape(Q, 4 * D).contiguous()
    ref = q4.gemv_f32(table, onehot).t().double()
    tol = 2 * (1e-4 * q4.gemv_f32(table.abs(), onehot).t().double() + 1e-6)
    del onehot, codes

    def one_pass():
        for c, o in zip(corpora, outs):
            q4.scan2(c, lut, out=o)

    results = []
    try:
        for cfg in scan_candidates():
            q4.scan2_set_config(*cfg)
            got = q4.scan2(corpora[0], lut)[:n].double()
            entry = {"config": list(cfg), "parity": bool(((got - ref).abs() <= tol).all())}
            if entry["parity"]:
                entry.update(_sample(one_pass, n_corpora, V * D // 4))
            results.append(entry)
    finally:
        q4.scan2_set_config(0, 0, 0, 0)
    best = _rank(results)
    del corpora, outs
    torch.cuda.empty_cache()
    default = next(r for r in results if r["config"] == [0, 0, 0, 0])
    return {"V": V, "Q": Q, "D": D, "corpora_cycled": n_corpora,
            "best": {"config": best["config"], "median_us": best["median_us"], "GBps": best["GBps"],
                     "default_us": default.get("median_us")},
            "candidates": results}


def tune(shapes=SHAPES, dev: torch.device | None = None, log=print, parts=("q4", "blocks", "scan"),
         block_shapes=BLOCK_SHAPES) -> dict:
    dev = dev or torch.device("cuda:0")
    q4.gemv_q4_clear_geometry()
    entries, block_entries, scan_entries = [], [], []
    for M, N, K, g in (shapes if "q4" in parts else []):
        t0 = time.time()
        e = tune_shape(M, N, K, g, dev)
        entries.append(e)
        b = e["best"]
        log(f"M{M} N{N} K{K} g{g}: best path {b['path']} waves {b['waves']} ksplit {b['ksplit']} "
            f"{b['median_us']:.3f} us ({b['GBps']:.0f} GB/s){' = default' if b['default'] else ''}; "
            f"{len(e['candidates'])} candidates, {time.time() - t0:.1f} s")
    for fmt in (q4.BLOCK_FORMATS if "blocks" in parts else []):
        for N, K in block_shapes:
            t0 = time.time()
            e = tune_block(fmt, N, K, dev)
            block_entries.append(e)
            b = e["best"]
            log(f"{fmt} N{N} K{K}: best {b['config']} {b['median_us']:.3f} us ({b['GBps']:.0f} GB/s), "
                f"default {b['default_us']:.3f} us; {len(e['candidates'])} candidates, "
                f"{time.time() - t0:.1f} s")
    if "scan" in parts:
        t0 = time.time()
        e = tune_scan(dev)
        scan_entries.append(e)
        b = e["best"]
        log(f"scan {e['V']}x{e['Q']} D{e['D']}: best {b['config']} {b['median_us']:.3f} us, "
            f"default {b['default_us']:.3f} us; {len(e['candidates'])} candidates, "
            f"{time.time() - t0:.1f} s")
    p = torch.cuda.get_device_properties(dev)
    return {"device": device_key(dev), "name": p.name, "arch": p.gcnArchName,
            "compute_units": p.multi_processor_count,
            "method": "parity-gated sweep; median of 25 samples of ~2 ms; cliff below 75% of best",
            "entries": entries, "block_entries": block_entries, "scan_entries": scan_entries}


def block_winners(prof: dict) -> dict:
    """Per format, the setting apply_profile applies: the same winner at
    every large shape tuned, at least APPLY_GAIN faster than the default
    there; formats without one are left out."""
    out = {}
    for fmt in q4.BLOCK_FORMATS:
        es = [e for e in prof.get("block_entries", []) if e["format"] == fmt
              and (e["N"], e["K"]) in BLOCK_LARGE]
        if len(es) != len(BLOCK_LARGE):
            continue
        cfgs = {tuple(e["best"]["config"]) for e in es}
        if len(cfgs) != 1 or cfgs == {(0, 0, 0)}:
            continue
        if all(_beats_default(e["best"]) for e in es):
            out[fmt] = cfgs.pop()
    return out


def scan_winner(prof: dict):
    """The scan setting apply_profile applies, or None."""
    for e in prof.get("scan_entries", []):
        b = e["best"]
        if b["config"] != [0, 0, 0, 0] and _beats_default(b):
            return tuple(b["config"])
    return None


def _beats_default(best: dict) -> bool:
    """The winner is APPLY_GAIN faster than the default (or the default
    failed its parity check and has no time)."""
    d = best.get("default_us")
    return d is None or d >= APPLY_GAIN * best["median_us"]


def apply_profile(path: str | None = None, dev: torch.device | None = None) -> int:
    """Load the profile for this device into the library; returns the number
    of settings made: gemv_q4 shapes whose winning geometry differs from the
    default plan, and the block-format and scan winners that hold (see
    block_winners, scan_winner).  A profile made on another device is refused."""
    path = path or default_profile_path(dev)
    prof = json.load(open(path))
    if prof["device"] != device_key(dev):
        raise ValueError(f"profile {path} is for {prof['device']}, this device is {device_key(dev)}")
    n = 0
    for e in prof["entries"]:
        b = e["best"]
        if not b["default"]:
            q4.gemv_q4_set_geometry(e["M"], e["N"], e["K"], e["group_size"], b["path"], b["waves"],
                                    b["ksplit"])
            n += 1
    for fmt, cfg in block_winners(prof).items():
        q4.gemv_block_set_config(fmt, *cfg)
        n += 1
    cfg = scan_winner(prof)
    if cfg is not None:
        q4.scan2_set_config(*cfg)
        n += 1
    return n


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out", default=None, help="profile path (default: tuned/<device>.json)")
    ap.add_argument("--quick", action="store_true",
                    help="only the one-row 4096 x 14336 shape (and the block formats' stream shape)")
    ap.add_argument("--only", default="q4,blocks,scan", help="comma list of q4, blocks, scan")
    args = ap.parse_args(argv)
    shapes = [(1, 14336, 4096, 128)] if args.quick else SHAPES
    prof = tune(shapes, log=lambda *a: print(*a, file=sys.stderr, flush=True),
                parts=tuple(args.only.split(",")),
                block_shapes=BLOCK_SHAPES[:1] if args.quick else BLOCK_SHAPES)
    out = args.out or default_profile_path()
    if os.path.exists(out):
        # parts not tuned in this run keep what the existing profile holds
        old = json.load(open(out))
        if old.get("device") == prof["device"]:
            for part, key in (("q4", "entries"), ("blocks", "block_entries"), ("scan", "scan_entries")):
                if part not in args.only.split(","):
                    prof[key] = old.get(key, [])
    os.makedirs(os.path.dirname(out), exist_ok=True)
    json.dump(prof, open(out, "w"), indent=1)
    print(out)
    return 0


if __name__ == "__main__":
    sys.exit(main())
