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
chunk positions per lane, x segments).

Reference: the library's dense fp32 GEMV on the device-dequantised weights,
with the bound |x| . |W|^T from the same GEMV of absolute values; a
candidate must agree within 2 (1e-4 bound + 1e-6).  Inputs are random and
generated on the device: codes and zero points uniform, scales uniform in
[0.002, 0.02], x ~ N(0, 1).

    python -m memory_bandwidth_amd.autotune [--out FILE] [--quick]

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
        y = q4.gemv_q4(self.x, m0["wq"], m0["scales"], m0["zeros"], g).double()
        return bool(((y - self.ref).abs() <= self.tol).all())

    def time(self) -> dict:
        """Median and p10-p90 per launch over SAMPLES replays of about SAMPLE_S each."""
        M, N, K, g = self.shape

        def one_pass():
            for m, y in zip(self.mats, self.ys):
                q4.gemv_q4(self.x, m["wq"], m["scales"], m["zeros"], g, out=y)

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
            samples.append(a.elapsed_time(b) * 1e-3 / (passes * self.n_mats))
        samples.sort()
        med = statistics.median(samples)
        return {"median_us": med * 1e6, "p10_us": samples[int(0.1 * (SAMPLES - 1))] * 1e6,
                "p90_us": samples[int(0.9 * (SAMPLES - 1))] * 1e6,
                "GBps": self.bytes / med / 1e9}


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
    timed = [r for r in results if r["parity"]]
    if not timed:
        raise RuntimeError(f"no configuration of {M}x{N}x{K} g{g} passed the parity check")
    best = min(timed, key=lambda r: r["median_us"])
    for r in timed:
        r["frac_of_best"] = best["median_us"] / r["median_us"]
        r["cliff"] = r["frac_of_best"] < CLIFF
    n_mats = case.n_mats
    del case
    torch.cuda.empty_cache()
    return {"M": M, "N": N, "K": K, "group_size": g, "matrices_cycled": n_mats,
            "best": {k: best[k] for k in ("path", "waves", "ksplit", "median_us", "p10_us",
                                          "p90_us", "GBps", "default")},
            "candidates": results}


def tune(shapes=SHAPES, dev: torch.device | None = None, log=print) -> dict:
    dev = dev or torch.device("cuda:0")
    q4.gemv_q4_clear_geometry()
    entries = []
    for M, N, K, g in shapes:
        t0 = time.time()
        e = tune_shape(M, N, K, g, dev)
        entries.append(e)
        b = e["best"]
        log(f"M{M} N{N} K{K} g{g}: best path {b['path']} waves {b['waves']} ksplit {b['ksplit']} "
            f"{b['median_us']:.3f} us ({b['GBps']:.0f} GB/s){' = default' if b['default'] else ''}; "
            f"{len(e['candidates'])} candidates, {time.time() - t0:.1f} s")
    p = torch.cuda.get_device_properties(dev)
    return {"device": device_key(dev), "name": p.name, "arch": p.gcnArchName,
            "compute_units": p.multi_processor_count,
            "method": "parity-gated sweep; median of 25 samples of ~2 ms; cliff below 75% of best",
            "entries": entries}


def apply_profile(path: str | None = None, dev: torch.device | None = None) -> int:
    """Load the profile for this device into the library; returns the number
    of shapes whose winning geometry differs from the default plan (those are
    the ones set).  A profile made on another device is refused."""
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
    return n


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out", default=None, help="profile path (default: tuned/<device>.json)")
    ap.add_argument("--quick", action="store_true", help="only the one-row 4096 x 14336 shape")
    args = ap.parse_args(argv)
    shapes = [(1, 14336, 4096, 128)] if args.quick else SHAPES
    prof = tune(shapes, log=lambda *a: print(*a, file=sys.stderr, flush=True))
    out = args.out or default_profile_path()
    os.makedirs(os.path.dirname(out), exist_ok=True)
    json.dump(prof, open(out, "w"), indent=1)
    print(out)
    return 0


if __name__ == "__main__":
    sys.exit(main())
