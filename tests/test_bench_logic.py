"""Host logic of the benchmark, checked with a fake timer (no GPU)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
import bench  # noqa: E402


def test_two_point_cancels_fixed_cost():
    C, T = 1.3e-3, 7.5e-6
    for n in (64, 256, 1024):
        assert bench.two_point(C + n * T, C + 2 * n * T, n) == pytest.approx(T, rel=1e-12)


def test_noise_rule():
    assert bench.resolvable(1.0, 1.2)
    assert not bench.resolvable(1.0, 1.19)
    assert not bench.resolvable(1.0, 0.9)
    # a fixed cost that dwarfs the work makes the cell noise
    C, T, n = 1e-3, 1e-7, 64
    assert not bench.resolvable(C + n * T, C + 2 * n * T)


def test_abba_orders_alternate():
    o = bench.abba_orders(["a", "b", "c"], 4)
    assert o == [["a", "b", "c"], ["c", "b", "a"], ["a", "b", "c"], ["c", "b", "a"]]


def test_sweep_discards_first_round_and_recovers_T():
    calls = []
    T = {"q": 5e-6, "f": 40e-6}

    def timer(k, n):
        calls.append((k, n))
        return 2e-4 + n * T[k]
    res = bench.sweep(timer, ["q", "f"], [64, 256], runs=3)
    # 4 rounds (1 discarded) x 2 kernels x 2 n x 2 points
    assert len(calls) == 4 * 2 * 2 * 2
    for k in T:
        assert len(res[k]["samples"]) == 3 * 2
        assert all(v == pytest.approx(T[k]) for v in res[k]["samples"])
        assert res[k]["noise"] == 0


def test_sweep_flags_noise_and_drift_is_cancelled_by_abba():
    clock = {"t": 0}

    def timer(k, n):
        clock["t"] += 1
        drift = 1 + 1e-4 * clock["t"]             # slow linear drift of the device
        if k == "tiny":
            return 1e-3 + n * 1e-9                 # unresolvable
        return (1e-3 + n * 1e-5) * drift
    res = bench.sweep(timer, ["tiny", "big"], [100], runs=4)
    assert res["tiny"]["noise"] == 4 and not res["tiny"]["samples"]
    med = bench.summarize(res["big"]["samples"])["median"]
    assert med == pytest.approx(1e-5, rel=2e-2)


def test_summarize_percentiles():
    s = bench.summarize([5.0, 1.0, 3.0, 2.0, 4.0])
    assert s["median"] == 3.0 and s["min"] == 1.0 and s["n"] == 5
    assert s["p10"] == pytest.approx(1.4) and s["p90"] == pytest.approx(4.6)
    assert bench.summarize([])["median"] is None


def test_traffic_is_null_when_kernel_changed(tmp_path, monkeypatch):
    p = tmp_path / "pmc.json"
    p.write_text(json.dumps({"kernel_source_sha256_16": "0" * 16,
                             "gemv_q4_hbm_bytes_per_launch": 123}))
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(p))
    assert bench.traffic_from_profile(1) is None
    p.write_text(json.dumps({"kernel_source_sha256_16": bench.kernel_source_hash(),
                             "gemv_q4_hbm_bytes_per_launch": 123}))
    assert bench.traffic_from_profile(1) == 123


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr


def test_cliffs_follow_the_80_percent_rule():
    sizes = [1, 2, 4, 8, 16, 32, 64]
    # rises (launch-bound), plateau, first cliff at 16, a new level, second cliff at 64
    best = [10, 50, 100, 95, 60, 58, 30]
    assert bench.find_cliffs(sizes, best) == [16, 64]
    assert bench.find_cliffs(sizes, [100, 81, 80.9, 80.5, 80.1, 80, 80]) == []
    assert bench.find_cliffs(sizes, [100, 79, 79, 79, 79, 79, 79]) == [2]
    assert [bench.cache_level(n, [16, 64]) for n in (1, 15, 16, 63, 64, 1000)] == [0, 0, 1, 1, 2, 2]
