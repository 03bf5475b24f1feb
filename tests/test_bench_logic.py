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


# ---------------------------------------------------------------- profile summaries

def _counter_csv(path, rows):
    """A rocprofv3 counter_collection.csv with the columns the summaries read."""
    cols = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name",
            "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w") as f:
        f.write(",".join(cols) + "\n")
        for r in rows:
            f.write(",".join(f'"{r[c]}"' if c == "Kernel_Name" else str(r[c]) for c in cols) + "\n")


FM = "void (anonymous namespace)::gemv_q4_fm_kernel<8, 8, 2, 16, 1, 8, 2, true>(float const*, int)"
SUM = "(anonymous namespace)::fm_sum_parts(float*, float const*, int, int, int)"
INT = "void (anonymous namespace)::gemv_q4_int_kernel<8, 64, 2, 4, 1, false, false, 16>(float const*)"
LM = "void (anonymous namespace)::gemv_q4_int_kernel<8, 32, 1, 4, 1, false, false, 16>(float const*)"
RR = "void (anonymous namespace)::read_reduce_kernel<true>(float const*, float*, long)"
WF = "void (anonymous namespace)::write_fill_kernel(float*, float, long)"


def _row(i, name, ctr, val, grid=131072, wg=512, us=10.0):
    return {"Dispatch_Id": i, "Kernel_Name": name, "Grid_Size": grid, "Workgroup_Size": wg,
            "Counter_Name": ctr, "Counter_Value": val, "Start_Timestamp": 1000 * i,
            "End_Timestamp": 1000 * i + int(us * 1000)}


def test_keyed_rows_tag_split_launches(tmp_path):
    """A multiply-add dispatch followed by fm_sum_parts is the K-split one;
    read_reduce is keyed with its grid."""
    _counter_csv(tmp_path / "p" / "run_counter_collection.csv", [
        _row(1, FM, "SQ_WAVES", 2048), _row(2, FM, "SQ_WAVES", 2048), _row(3, SUM, "SQ_WAVES", 128),
        _row(4, RR, "SQ_WAVES", 64, grid=524288, wg=256), _row(5, FM, "SQ_WAVES", 2048)])
    keys = [k for k, _ in bench._keyed_rows(str(tmp_path / "p"))]
    fm = "gemv_q4_fm_kernel<8, 8, 2, 16, 1, 8, 2, true>"
    assert keys == [fm, fm + " K split", "fm_sum_parts", "read_reduce_kernel<true> grid 524288", fm]


def test_summarize_pmc_scales_by_the_probes(tmp_path, monkeypatch):
    """FETCH_SIZE is scaled so the 2 GiB read probe reads its own size, WRITE_SIZE so
    write_fill writes its own; the stream kernel is the gemv_q4 kernel with the
    most dispatches, and its bytes per launch land in the JSON bench.py reads."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(tmp_path / "profiles" / "pmc.json"))
    (tmp_path / "profiles").mkdir()
    probe_kib = bench.wl.PROBE_BYTES / 1024
    fetch = [_row(1, RR, "FETCH_SIZE", probe_kib / 2, grid=1048576, wg=256),    # counter reads half
             _row(2, WF, "FETCH_SIZE", 1.0)]
    write = [_row(1, RR, "WRITE_SIZE", 1.0, grid=1048576, wg=256),
             _row(2, WF, "WRITE_SIZE", probe_kib)]
    for i in range(3, 3 + 64):
        fetch.append(_row(i, INT, "FETCH_SIZE", 15000.0))
        write.append(_row(i, INT, "WRITE_SIZE", 64.0))
    fetch.append(_row(99, FM, "FETCH_SIZE", 16000.0))
    write.append(_row(99, FM, "WRITE_SIZE", 400.0))
    lm_kib = bench.wl.q4_weight_bytes(bench.wl.LM_HEAD.N, bench.wl.LM_HEAD.K, bench.wl.LM_HEAD.g) / 1024 / 2
    for i in range(100, 108):     # the LM head kernel: fewer dispatches, not taken for the stream
        fetch.append(_row(i, LM, "FETCH_SIZE", lm_kib))
        write.append(_row(i, LM, "WRITE_SIZE", 593.5))
    _counter_csv(tmp_path / "f" / "run_counter_collection.csv", fetch)
    _counter_csv(tmp_path / "w" / "run_counter_collection.csv", write)
    out = bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), "t", "cmd")
    assert "(the LM head 896 -> 151936 g32, 78702848 B): 78702848 B fetched, ratio 1.0000" in open(out).read()
    j = json.load(open(tmp_path / "profiles" / "pmc.json"))
    assert j["fetch_factor"] == pytest.approx(2.0) and j["write_factor"] == pytest.approx(1.0)
    assert j["kernel"].startswith("gemv_q4_int_kernel<8, 64")
    assert j["gemv_q4_fetch_bytes_per_launch"] == round(15000.0 * 1024 * 2)
    assert j["gemv_q4_write_bytes_per_launch"] == 64 * 1024
    assert j["kernel_source_sha256_16"] == bench.kernel_source_hash()


def test_summarize_counters_derived_lines(tmp_path, monkeypatch):
    """Counters of several passes merge per kernel; the VALU issue rate, the LDS
    busy share of the dispatch's CU cycles and the FMA share are derived from them."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    us = 20.0
    p1 = [_row(1, INT, "SQ_WAVES", 4096, us=us), _row(1, INT, "SQ_INSTS_VALU", 4096 * 500, us=us)]
    cyc = bench.CUS * us * 1e3 * bench.CLOCK_GHZ
    p5 = [_row(1, INT, "SQ_LDS_IDX_ACTIVE", 0.25 * cyc, us=us),
          _row(1, INT, "SQ_INSTS_VALU_FMA_F32", 4096 * 100, us=us),
          _row(1, INT, "SQ_LDS_BANK_CONFLICT", 7, us=us)]
    _counter_csv(tmp_path / "a" / "run_counter_collection.csv", p1)
    _counter_csv(tmp_path / "b" / "run_counter_collection.csv", p5)
    out = bench.summarize_counters([str(tmp_path / "a"), str(tmp_path / "b")], "c", "cmd")
    text = open(out).read()
    assert "VALU: 500 wavefront-instructions per wavefront" in text
    assert f"{4096 * 500 / (bench.SIMDS * us * 1e3):.3f} issued per SIMD per ns" in text
    assert "LDS busy 25.0% of the dispatch's CU cycles" in text and "bank-conflict cycles 7" in text
    assert "fp32 FMA 20.0% of the VALU instructions" in text


def test_with_floor_records_the_fraction():
    """A streaming cell carries the read floor of its own size and its share of it."""
    rec = {"us_per_launch": {"median": 10.0}}
    out = bench.with_floor(rec, {"stats": {"median": 8e-6}})
    assert out["single_launch_floor_us"] == 8.0 and out["frac_of_single_launch_floor"] == 0.8
    assert "single_launch_floor_us" not in rec
