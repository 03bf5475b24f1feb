"""C-ABI checks that need no GPU: the library loads, exports every function
include/q4gemv.h, include/q4blocks.h and include/q4scan.h declare, and rejects bad arguments before touching the
device.  Calls here either fail validation or stop at the device check; none
launches a kernel."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("q4gemv.h", "q4blocks.h", "q4scan.h")]

import memory_bandwidth_amd as q4  # noqa: E402
import workloads  # noqa: E402


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(q4.LIB_PATH):
        from memory_bandwidth_amd import build
        build.build()
    return q4.lib()


def _gpu_present() -> bool:
    import torch
    return torch.cuda.is_available()


def header_functions():
    names = []
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names += re.findall(r"^(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return names


def test_header_declares_expected_functions():
    assert sorted(header_functions()) == sorted(q4.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    out = subprocess.run(["nm", "-D", "--defined-only", q4.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in header_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_abi_version_and_strerror(L):
    assert q4.abi_version() == 1
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(q4.strerror(code), str) and q4.strerror(code)


A16 = 0x10000          # fake, aligned, never dereferenced device addresses
A16B = 0x20000


@pytest.mark.parametrize("M,N,K,g,want", [
    (0, 8, 128, 32, q4.Q4_EINVAL), (9, 8, 128, 32, q4.Q4_EINVAL),
    (1, -1, 128, 32, q4.Q4_EINVAL), (1, 8, 0, 32, q4.Q4_EINVAL),
    (1, 8, 96, 64, q4.Q4_EINVAL), (1, 8, 160, 128, q4.Q4_EINVAL),
    (1, 8, 100, 32, q4.Q4_EINVAL), (1, 8, 64, 128, q4.Q4_EINVAL),
    (1, 0, 128, 32, q4.Q4_OK),      # empty output: nothing launched
])
def test_gemv_q4_shape_validation(L, M, N, K, g, want):
    assert L.gemv_q4(A16, A16, A16, A16, A16, M, N, K, g, None) == want


def test_gemv_q4_pointer_validation(L):
    assert L.gemv_q4(None, A16, A16, A16, A16, 1, 8, 128, 32, None) == q4.Q4_ENULL
    assert L.gemv_q4(A16, A16, A16, None, A16, 1, 8, 128, 32, None) == q4.Q4_ENULL
    assert L.gemv_q4(A16 + 4, A16, A16, A16, A16, 1, 8, 128, 32, None) == q4.Q4_EALIGN
    assert L.gemv_q4(A16, A16 + 8, A16, A16, A16, 1, 8, 128, 32, None) == q4.Q4_EALIGN
    assert L.gemv_q4(A16, A16, A16 + 1, A16, A16, 1, 8, 128, 32, None) == q4.Q4_EALIGN
    assert L.gemv_q4(A16, A16, A16, A16, A16 + 2, 1, 8, 128, 32, None) == q4.Q4_EALIGN
    # zeros need only byte alignment (a valid call: it would launch on a GPU
    # host, where these fake addresses must never reach a kernel)
    if not _gpu_present():
        assert L.gemv_q4(A16, A16, A16, A16 + 1, A16, 1, 8, 128, 32, None) == q4.Q4_EDEVICE


def test_gemv_q4_swiglu_validation(L):
    f = L.gemv_q4_swiglu
    assert f(A16, A16, A16, A16, A16, A16, A16, A16, 9, 8, 128, 32, None) == q4.Q4_EINVAL
    assert f(A16, A16, A16, A16, A16, A16, A16, A16, 1, 8, 100, 32, None) == q4.Q4_EINVAL
    assert f(A16, A16, A16, A16, A16, A16, A16, A16, 1, 0, 128, 32, None) == q4.Q4_OK
    assert f(A16, A16, A16, A16, None, A16, A16, A16, 1, 8, 128, 32, None) == q4.Q4_ENULL
    assert f(A16, A16, A16, A16, A16, A16, None, A16, 1, 8, 128, 32, None) == q4.Q4_ENULL
    assert f(A16, A16, A16, A16, A16 + 8, A16, A16, A16, 1, 8, 128, 32, None) == q4.Q4_EALIGN
    assert f(A16, A16, A16, A16, A16, A16 + 1, A16, A16, 1, 8, 128, 32, None) == q4.Q4_EALIGN
    assert f(A16, A16, A16, A16, A16, A16, A16, A16 + 2, 1, 8, 128, 32, None) == q4.Q4_EALIGN


def test_other_entry_points_validation(L):
    assert L.gemv_f32(A16, A16, A16, 1, 8, 6, None) == q4.Q4_EINVAL
    assert L.gemv_f32(A16, A16, A16, 0, 8, 8, None) == q4.Q4_EINVAL
    assert L.gemv_f32(A16, A16, A16, 1, 0, 8, None) == q4.Q4_OK
    assert L.gemv_f32(A16 + 4, A16, A16, 1, 8, 8, None) == q4.Q4_EALIGN
    assert L.dequant_q4(A16, A16, A16, None, None, 4, 64, 32, None) == q4.Q4_ENULL
    assert L.dequant_q4(A16, A16, A16, A16 + 4, None, 4, 64, 32, None) == q4.Q4_EALIGN
    assert L.dequant_q4(A16, A16, A16, None, A16 + 4, 4, 64, 32, None) == q4.Q4_EALIGN
    assert L.dequant_q4(A16, A16, A16, A16, None, 4, 96, 128, None) == q4.Q4_EINVAL
    assert L.read_reduce(A16, 6, A16B, 4, None) == q4.Q4_EINVAL
    assert L.read_reduce(A16, 8, A16B, 0, None) == q4.Q4_EINVAL
    assert L.read_reduce(A16, 8, A16B, 65537, None) == q4.Q4_EINVAL
    assert L.read_reduce(A16 + 4, 8, A16B, 4, None) == q4.Q4_EALIGN
    assert L.read_reduce(A16, 8, None, 4, None) == q4.Q4_ENULL
    assert L.write_fill(A16, 6, ctypes.c_float(1.0), 0, None) == q4.Q4_EINVAL
    assert L.write_fill(A16 + 8, 8, ctypes.c_float(1.0), 0, None) == q4.Q4_EALIGN
    assert L.write_fill(None, 0, ctypes.c_float(1.0), 0, None) == q4.Q4_OK
    for passes in (0, -1, 4097):
        assert L.read_reduce_passes(A16, 8, passes, A16B, 4, None) == q4.Q4_EINVAL
        assert L.copy_vec4(A16, A16B, 8, passes, 0, None) == q4.Q4_EINVAL
    assert L.read_reduce_passes(A16, 6, 2, A16B, 4, None) == q4.Q4_EINVAL
    assert L.read_reduce_passes(A16 + 4, 8, 2, A16B, 4, None) == q4.Q4_EALIGN
    assert L.copy_vec4(A16, A16B, 6, 1, 0, None) == q4.Q4_EINVAL
    assert L.copy_vec4(A16, A16B, 8, 1, 65537, None) == q4.Q4_EINVAL
    assert L.copy_vec4(A16, A16B, 8, 1, -1, None) == q4.Q4_EINVAL
    assert L.copy_vec4(None, A16B, 8, 1, 0, None) == q4.Q4_ENULL
    assert L.copy_vec4(A16, A16B + 8, 8, 1, 0, None) == q4.Q4_EALIGN
    assert L.copy_vec4(A16, A16 + 16, 8, 1, 0, None) == q4.Q4_EINVAL     # overlapping ranges
    assert L.copy_vec4(A16 + 16, A16, 8, 1, 0, None) == q4.Q4_EINVAL
    assert L.copy_vec4(None, None, 0, 1, 0, None) == q4.Q4_OK


def test_no_device_reports_edevice(L):
    """On a host without a gfx950 GPU, a valid call stops at the device check."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert L.gemv_q4(A16, A16, A16, A16, A16, 1, 8, 128, 32, None) == q4.Q4_EDEVICE
    assert L.gemv_q4_swiglu(A16, A16, A16, A16, A16, A16, A16, A16, 1, 8, 128, 32, None) == q4.Q4_EDEVICE
    assert L.read_reduce(A16, 8, A16B, 4, None) == q4.Q4_EDEVICE
    assert L.copy_vec4(A16, A16B, 8, 1, 0, None) == q4.Q4_EDEVICE


SHAPES = ([workloads.SMALL_896, workloads.LM_HEAD, workloads.STREAM_SHAPE]
          + list(workloads.DECODER_LAYER) + [s for M in (1, 4, 8) for s in workloads.ffn_8b(M)])


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s.label}" for s in SHAPES])
def test_geometry_covers_every_row(shape):
    geo = q4.gemv_q4_geometry(shape.M, shape.N, shape.K, shape.g)
    lpr, S = geo["lanes_per_row"], geo["ksplit"]
    integer = q4.gemv_q4_path(shape.M, shape.N, shape.K, shape.g) == q4.Q4_PATH_INTEGER
    fm = not integer and shape.M > 1      # the fp32 multiply-add kernel
    assert lpr in (16, 32, 64) and S in (1, 2, 4)
    assert geo["block"] in ((256, 512, 1024) if integer else ((512,) if fm else (256,)))
    waves = geo["block"] // 64
    rows_per_wg = geo["rows_per_wave"] * waves // S
    C = shape.K // 32
    if integer or fm:
        # each workgroup owns ceil(N / grid) rows, at most rows_per_wave per row group
        rpg = -(-shape.N // geo["grid"])
        assert rpg <= rows_per_wg and geo["grid"] * rpg >= shape.N > (geo["grid"] - 1) * rpg
    seg = -(-C // geo["segments"])
    if integer and shape.M == 1:
        # 144-byte records and 128 bytes of residual slots per chunk of the whole x
        assert geo["segments"] == 1 and C * 272 + waves * geo["rows_per_wave"] * 4 <= 160 * 1024
        # a lane holds at most 3 chunk positions of its K slice
        assert -(-C // S) <= 3 * 64
    elif integer:
        # M rows of 144-byte records and pool slots per segment, within the CU's LDS
        mp = 2 if shape.M <= 2 else (4 if shape.M <= 4 else 8)
        assert shape.M * seg * 152 + waves * geo["rows_per_wave"] * mp * 4 <= 160 * 1024
        assert -(-seg // S) <= 2 * 64
    elif fm:
        # M rows of 144-byte staged chunks per segment and the partial sums, within the LDS;
        # at most 16 chunk positions per lane (8 for 7 and 8 rows)
        assert shape.M * seg * 144 + waves * geo["rows_per_wave"] * shape.M * 4 <= 160 * 1024
        part = -(-seg // S)
        assert lpr == 16 and -(-part // 16) <= (8 if shape.M >= 7 else 16)
    else:
        assert geo["grid"] * rows_per_wg >= shape.N > (geo["grid"] - 1) * rows_per_wg
        seg = -(-C // geo["segments"])
        # x segment fits the 64 KiB LDS budget
        assert shape.M * seg * 128 <= 64 * 1024


PATHS = [
    # M, N, K, g, path: one activation row with more than 16 chunks per row takes the integer path
    (1, 14336, 4096, 128, 1), (1, 4096, 14336, 128, 1), (1, 65, 2048, 128, 1),
    (1, 1, 18688, 128, 1), (1, 1, 19200, 128, 1), (1, 4, 19328, 128, 0), (1, 2, 19264, 32, 1),
    (1, 4096, 19232, 32, 1), (1, 4096, 19264, 32, 0), (1, 896, 896, 32, 1), (1, 151936, 896, 32, 1),
    (1, 63, 2016, 32, 1), (1, 7, 1024, 32, 1), (1, 9, 512, 32, 0), (1, 9, 544, 32, 1),
    # 2 to 8 activation rows take the fp32 multiply-add path (the integer one only on request)
    (2, 14336, 4096, 128, 0), (8, 4096, 14336, 128, 0),
    (4, 896, 896, 32, 0), (2, 64, 1024, 32, 0), (3, 4864, 896, 32, 0), (7, 100, 2048, 128, 0),
    (4, 4096, 14336, 128, 0), (2, 4096, 14336, 128, 0), (2, 300, 8192, 128, 0),
]


@pytest.mark.parametrize("M,N,K,g,path", PATHS, ids=[f"M{a}N{b}K{c}g{d}" for a, b, c, d, _ in PATHS])
def test_arithmetic_path(M, N, K, g, path):
    assert q4.gemv_q4_path(M, N, K, g) == path


def test_integer_geometry_balances_cus():
    """14336 rows at M = 1: 512 workgroups of 8 wavefronts and 28 rows (2 per
    CU), not 448 of 32; the 14336 -> 4096 projection splits K four ways and
    takes one 16-wavefront workgroup of 16 rows per CU."""
    geo = q4.gemv_q4_geometry(1, 14336, 4096, 128)
    assert geo["grid"] == 512 and geo["block"] == 512 and geo["ksplit"] == 1
    geo = q4.gemv_q4_geometry(1, 4096, 14336, 128)
    assert geo["grid"] == 256 and geo["block"] == 1024 and geo["ksplit"] == 4


@pytest.mark.parametrize("N,K", [(896, 4864), (2048, 2048), (65, 2048)])
def test_integer_geometry_small_n_keeps_small_workgroups(N, K):
    """Too few rows to give every CU an 8-wavefront workgroup: 4 wavefronts."""
    geo = q4.gemv_q4_geometry(1, N, K, 128 if K % 128 == 0 else 32)
    assert geo["block"] == 256


def test_geometry_rejects_bad_shapes():
    with pytest.raises(q4.Q4Error):
        q4.gemv_q4_geometry(1, 8, 100, 32)
    with pytest.raises(q4.Q4Error):
        q4.gemv_q4_path(1, 8, 100, 32)


# ---------------------------------------------------------------- geometry overrides

@pytest.fixture
def clean_geometry():
    q4.gemv_q4_clear_geometry()
    yield
    q4.gemv_q4_clear_geometry()


@pytest.mark.parametrize("M,N,K,g,split", [
    (8, 4096, 14336, 128, True), (4, 4096, 14336, 128, True), (3, 300, 14336, 128, True),
    (2, 4096, 14336, 128, False),     # x in one segment: no split
    (8, 14336, 4096, 128, False),     # likewise
    (1, 4096, 14336, 128, False),     # one row: the integer path
    (8, 16384, 14336, 128, False),    # too many rows per CU for the split to pay
])
def test_workspace_size(M, N, K, g, split):
    n = q4.gemv_q4_workspace_size(M, N, K, g)
    if split:
        assert n > 0 and n % (4 * M * N) == 0 and 2 <= n // (4 * M * N) <= 8
    else:
        assert n == 0
    assert q4.gemv_q4_workspace_size(M, 0, K, g) == 0


def test_static_array_holds_every_planned_workspace():
    """gemv_q4_static's 512 KiB array must cover every K split the planner
    makes, or the entry point would refuse shapes gemv_q4_ws serves."""
    rng = np.random.default_rng(8)
    shapes = [(M, N, K, g) for M in range(1, 9) for g in (32, 128)
              for N in (1, 64, 896, 2048, 2049, 4096, 8192, 16384, 151936)
              for K in (g, 1024, 4096, 14336, 16384, 28672, 1 << 20) if K % g == 0]
    for _ in range(3000):
        g = int(rng.choice([32, 128]))
        shapes.append((int(rng.integers(1, 9)), int(rng.integers(1, 300000)), g * int(rng.integers(1, 2049)), g))
    worst = max(q4.gemv_q4_workspace_size(*s) for s in shapes)
    assert 0 < worst <= 512 * 1024


def test_workspace_entry_points_validate(L):
    n = ctypes.c_size_t()
    assert L.gemv_q4_workspace_size(1, 8, 100, 32, ctypes.byref(n)) == q4.Q4_EINVAL
    assert L.gemv_q4_workspace_size(8, 4096, 14336, 128, None) == q4.Q4_ENULL
    assert L.gemv_q4_ws(A16, A16, A16, A16, A16, 1, 8, 100, 32, A16B, 64, None) == q4.Q4_EINVAL
    assert L.gemv_q4_ws(A16, A16, A16, A16, A16, 8, 0, 14336, 128, None, 0, None) == q4.Q4_OK
    assert L.gemv_q4_ws(A16, A16, A16, A16, A16, 8, 64, 14336, 128, A16B + 4, 64, None) == q4.Q4_EALIGN
    assert L.gemv_q4_ws(None, A16, A16, A16, A16, 8, 64, 14336, 128, A16B, 64, None) == q4.Q4_ENULL


def test_set_geometry_changes_the_plan(clean_geometry):
    M, N, K, g = 1, 14336, 4096, 128
    default = q4.gemv_q4_geometry(M, N, K, g)
    q4.gemv_q4_set_geometry(M, N, K, g, q4.Q4_PATH_INTEGER, waves=4, ksplit=2)
    geo = q4.gemv_q4_geometry(M, N, K, g)
    assert geo["block"] == 256 and geo["ksplit"] == 2 and geo != default
    assert q4.gemv_q4_path(M, N, K, g) == q4.Q4_PATH_INTEGER
    q4.gemv_q4_set_geometry(M, N, K, g, q4.Q4_PATH_FMA)            # replaces the entry
    assert q4.gemv_q4_path(M, N, K, g) == q4.Q4_PATH_FMA
    assert q4.gemv_q4_path(M, N + 1, K, g) == q4.Q4_PATH_INTEGER  # other shapes keep the plan
    q4.gemv_q4_clear_geometry()
    assert q4.gemv_q4_geometry(M, N, K, g) == default


@pytest.mark.parametrize("M,N,K,g,path,waves,ksplit", [
    (1, 896, 512, 32, 1, 0, 0),          # integer path needs K > 512 (32 or 64 lanes per row)
    (1, 896, 896, 32, 1, 0, 2),          # 32-lane rows: no K-split
    (1, 64, 32768, 128, 1, 0, 1),        # 1024 chunks on one wavefront: > 3 per lane
    (1, 64, 4096, 128, 1, 4, 8),         # ksplit not in {1, 2, 4}
    (1, 64, 4096, 128, 0, 8, 0),         # the multiply-add path has 4 wavefronts
    (4, 64, 4096, 128, 1, 16, 0),        # 2..4 rows use 8 wavefronts
    (4, 64, 4096, 128, 0, 4, 0),         # so does the multiply-add path for 2..8 rows
    (8, 64, 4096, 128, 0, 16, 0),
    (2, 64, 1024, 32, 1, 0, 0),          # the integer path for several rows needs K > 1024
    (1, 64, 4096, 128, 2, 0, 0),         # no such path
    (1, 64, 100, 32, 0, 0, 0),           # invalid shape
])
def test_set_geometry_rejects_what_cannot_run(clean_geometry, M, N, K, g, path, waves, ksplit):
    valid = K % g == 0
    before = q4.gemv_q4_geometry(M, N, K, g) if valid else None
    with pytest.raises(q4.Q4Error):
        q4.gemv_q4_set_geometry(M, N, K, g, path, waves, ksplit)
    if valid:
        assert q4.gemv_q4_geometry(M, N, K, g) == before   # plan unchanged


def test_set_geometry_table_limit(clean_geometry):
    for n in range(256):
        q4.gemv_q4_set_geometry(1, 100 + n, 4096, 128, q4.Q4_PATH_FMA)
    with pytest.raises(q4.Q4Error):
        q4.gemv_q4_set_geometry(1, 99, 4096, 128, q4.Q4_PATH_FMA)
    q4.gemv_q4_set_geometry(1, 100, 4096, 128, q4.Q4_PATH_INTEGER)   # replacing still works


def test_tuned_profile_is_well_formed_and_applies(clean_geometry):
    """The committed profile names its device and, for every shape, a winner
    that passed parity and that the library accepts; cliffs are flagged."""
    import json
    import os
    from memory_bandwidth_amd import autotune
    files = [f for f in os.listdir(autotune.TUNED_DIR) if f.endswith(".json")]
    assert files
    for f in files:
        prof = json.load(open(os.path.join(autotune.TUNED_DIR, f)))
        assert f == prof["device"] + ".json"
        for e in prof["entries"]:
            b = e["best"]
            timed = [c for c in e["candidates"] if c["parity"]]
            assert b["median_us"] == min(c["median_us"] for c in timed)
            assert all(c["cliff"] == (c["frac_of_best"] < autotune.CLIFF) for c in timed)
            q4.gemv_q4_set_geometry(e["M"], e["N"], e["K"], e["group_size"], b["path"],
                                    b["waves"], b["ksplit"])
        for e in prof.get("block_entries", []) + prof.get("scan_entries", []):
            timed = [c for c in e["candidates"] if c["parity"]]
            assert e["best"]["median_us"] == min(c["median_us"] for c in timed)
            assert all(c["cliff"] == (c["frac_of_best"] < autotune.CLIFF) for c in timed)
        try:
            for e in prof.get("block_entries", []):
                q4.gemv_block_set_config(e["format"], *e["best"]["config"])
            for e in prof.get("scan_entries", []):
                q4.scan2_set_config(*e["best"]["config"])
        finally:
            for fmt in q4.BLOCK_FORMATS:
                q4.gemv_block_set_config(fmt, 0, 0, 0)
            q4.scan2_set_config(0, 0, 0, 0)


def test_profile_winner_rules():
    """A block-format winner applies only when it wins at both large shapes
    by at least 3%; the scan's only when it beats the default by 3%."""
    from memory_bandwidth_amd import autotune

    def be(fmt, shape, cfg, us, default_us):
        return {"format": fmt, "N": shape[0], "K": shape[1],
                "best": {"config": list(cfg), "median_us": us, "default_us": default_us}}

    big, lm = autotune.BLOCK_LARGE
    prof = {"block_entries": [be("q4_0", big, (2, 4, 1), 9.0, 10.0), be("q4_0", lm, (2, 4, 1), 9.0, 9.5),
                              be("q8_0", big, (1, 4, 2), 9.0, 10.0), be("q8_0", lm, (2, 4, 2), 9.0, 10.0),
                              be("q4_k", big, (1, 8, 2), 9.0, 9.1), be("q4_k", lm, (1, 8, 2), 9.0, 10.0),
                              be("q6_k", big, (0, 0, 0), 9.0, 9.0), be("q6_k", lm, (0, 0, 0), 9.0, 9.0)],
            "scan_entries": [{"best": {"config": [1, 1, 256, 2], "median_us": 10.0, "default_us": 10.4}}]}
    assert autotune.block_winners(prof) == {"q4_0": (2, 4, 1)}
    assert autotune.scan_winner(prof) == (1, 1, 256, 2)
    prof["scan_entries"][0]["best"]["default_us"] = 10.2
    assert autotune.scan_winner(prof) is None
    prof["scan_entries"][0]["best"]["default_us"] = None      # the default failed parity
    assert autotune.scan_winner(prof) == (1, 1, 256, 2)


def test_block_and_scan_validation(L):
    IP = ctypes.POINTER(ctypes.c_int)
    e, b = ctypes.c_int(), ctypes.c_int()
    assert L.block_geometry(3, ctypes.byref(e), ctypes.byref(b)) == q4.Q4_OK and (e.value, b.value) == (256, 144)
    assert L.block_geometry(0, ctypes.byref(e), ctypes.byref(b)) == q4.Q4_EINVAL
    assert L.block_geometry(1, None, ctypes.byref(b)) == q4.Q4_ENULL
    assert L.gemv_block(1, A16, A16, A16, 2, 8, 256, None) == q4.Q4_EINVAL      # M != 1
    assert L.gemv_block(1, A16, A16, A16, 1, 8, 320, None) == q4.Q4_EINVAL      # K % 256
    assert L.gemv_block(1, A16, A16, A16, 1, 8, 32768 + 256, None) == q4.Q4_EINVAL
    assert L.gemv_block(6, A16, A16, A16, 1, 8, 256, None) == q4.Q4_EINVAL      # format
    assert L.gemv_block(1, A16, A16, A16, 1, 0, 256, None) == q4.Q4_OK          # empty
    assert L.gemv_block(1, None, A16, A16, 1, 8, 256, None) == q4.Q4_ENULL
    assert L.gemv_block(1, A16 + 4, A16, A16, 1, 8, 256, None) == q4.Q4_EALIGN
    assert L.gemv_block(1, A16, A16 + 8, A16, 1, 8, 256, None) == q4.Q4_EALIGN
    assert L.dequant_block(2, A16, A16 + 4, 8, 256, None) == q4.Q4_EALIGN
    assert L.dequant_block(2, A16, None, 8, 256, None) == q4.Q4_ENULL
    assert L.gemv_block_set_config(5, 4, 4, 0) == q4.Q4_EINVAL                 # Q6_K spills at R = 4
    assert L.gemv_block_set_config(1, 3, 4, 0) == q4.Q4_EINVAL
    assert L.gemv_block_set_config(1, 2, 8, 65) == q4.Q4_EINVAL
    r, w, g = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    assert L.gemv_block_set_config(1, 2, 8, 3) == q4.Q4_OK
    assert L.gemv_block_config(1, ctypes.byref(r), ctypes.byref(w), ctypes.byref(g)) == q4.Q4_OK
    assert (r.value, w.value, g.value) == (2, 8, 3)
    assert L.gemv_block_set_config(1, 0, 0, 0) == q4.Q4_OK
    assert L.scan2(A16, A16, A16, 8, 768, 9, None) == q4.Q4_EINVAL              # Q > 8
    assert L.scan2(A16, A16, A16, 8, 96, 8, None) == q4.Q4_EINVAL               # D % 64
    assert L.scan2(A16, A16, A16, 8, 2048, 8, None) == q4.Q4_EINVAL             # LDS table limit
    assert L.scan2(A16, A16, A16, 0, 768, 8, None) == q4.Q4_OK
    assert L.scan2(None, A16, A16, 8, 768, 8, None) == q4.Q4_ENULL
    assert L.scan2(A16 + 4, A16, A16, 8, 768, 8, None) == q4.Q4_EALIGN
    assert L.scan2_set_config(0, 1, 256, 1) == q4.Q4_OK                        # table in memory
    if not _gpu_present():                      # a valid call: never launched on fake addresses
        assert L.scan2(A16, A16, A16, 8, 2048, 8, None) == q4.Q4_EDEVICE
    assert L.scan2_set_config(1, 3, 256, 1) == q4.Q4_EINVAL
    assert L.scan2_set_config(1, 1, 256, 16) == q4.Q4_EINVAL
    assert L.scan2_set_config(0, 0, 0, 0) == q4.Q4_OK
    t = ctypes.c_int()
    assert L.scan2_config(ctypes.byref(r), ctypes.byref(w), ctypes.byref(g), ctypes.byref(t)) == q4.Q4_OK
    assert (r.value, w.value, g.value, t.value) == (1, 1, 1024, 0)


def test_tuner_candidates_are_what_the_library_accepts():
    """Host-only: the block-format candidates are exactly the settings the
    library accepts (R = 4 only where it compiles without spilling), plus the
    default; the scan's are the LDS-table grid plus the page's tail with the
    table in memory and the default."""
    from memory_bandwidth_amd import autotune
    for fmt in q4.BLOCK_FORMATS:
        cands = autotune.block_candidates(fmt)
        assert cands[0] == (0, 0, 0) and len(set(cands)) == len(cands)
        r4 = fmt not in ("q5_k", "q6_k")
        assert len(cands) == 1 + (3 if r4 else 2) * 2 * 4
    cs = autotune.scan_candidates()
    assert len(cs) == 26 and cs[0] == (0, 0, 0, 0) and (0, 1, 256, 1) in cs
    for c in cs[1:]:
        q4.scan2_set_config(*c)
    q4.scan2_set_config(0, 0, 0, 0)
    assert q4.scan2_config() == (1, 1, 1024, 0)


# ---------------------------------------------------------------- limits and concurrent callers

def test_k_limit_rejected_before_anything_runs():
    """K past 2^24 would need byte offsets beyond the kernels' 32-bit buffer
    addressing: every entry point returns Q4_EINVAL for it (host-only query;
    the launch entry points validate the same way before touching a device)."""
    assert q4.gemv_q4_path(1, 8, 1 << 24, 128) in (q4.Q4_PATH_FMA, q4.Q4_PATH_INTEGER)
    for fn in (lambda: q4.gemv_q4_path(1, 8, (1 << 24) + 128, 128),
               lambda: q4.gemv_q4_geometry(8, 4, (1 << 24) + 128, 128),
               lambda: q4.gemv_q4_set_geometry(1, 8, (1 << 24) + 128, 128, q4.Q4_PATH_FMA, 0, 0)):
        with pytest.raises(q4.Q4Error) as e:
            fn()
        assert e.value.status == q4.Q4_EINVAL
    L = q4.lib()
    assert L.gemv_q4(None, None, None, None, None, 1, 8, (1 << 24) + 128, 128, None) == q4.Q4_EINVAL


def test_large_matrices_keep_their_geometry():
    """Shapes whose scale or code arrays pass 4 GiB from a wavefront's first
    row (ranges once formed in 32 bits) plan like any other: the ranges are
    64-bit and clamped, and a wavefront only reads its own rows."""
    for M, N, K, g in [(1, 1 << 21, 65536, 32), (1, (1 << 22) + 3, 4096, 32), (8, 1 << 20, 1 << 16, 128)]:
        geo = q4.gemv_q4_geometry(M, N, K, g)
        assert geo["grid"] >= 1 and geo["lanes_per_row"] in (16, 32, 64)


def test_geometry_table_is_safe_beside_concurrent_readers():
    """One thread flips a shape's override between two settings while others
    read its geometry: every read is one of the two settings' geometries or
    the default plan's (never a mix)."""
    import threading
    M, N, K, g = 1, 14336, 4096, 128
    q4.gemv_q4_clear_geometry()
    default = q4.gemv_q4_geometry(M, N, K, g)
    q4.gemv_q4_set_geometry(M, N, K, g, q4.Q4_PATH_INTEGER, 4, 0)
    a = q4.gemv_q4_geometry(M, N, K, g)
    q4.gemv_q4_set_geometry(M, N, K, g, q4.Q4_PATH_FMA, 0, 2)
    b = q4.gemv_q4_geometry(M, N, K, g)
    allowed = [default, a, b]
    assert a != b
    stop = threading.Event()
    bad = []

    def writer():
        i = 0
        while not stop.is_set():
            if i % 3 == 2:
                q4.gemv_q4_clear_geometry()
            elif i % 2:
                q4.gemv_q4_set_geometry(M, N, K, g, q4.Q4_PATH_INTEGER, 4, 0)
            else:
                q4.gemv_q4_set_geometry(M, N, K, g, q4.Q4_PATH_FMA, 0, 2)
            i += 1

    def reader():
        for _ in range(3000):
            geo = q4.gemv_q4_geometry(M, N, K, g)
            if geo not in allowed:
                bad.append(geo)

    try:
        w = threading.Thread(target=writer)
        rs = [threading.Thread(target=reader) for _ in range(3)]
        w.start()
        for r in rs:
            r.start()
        for r in rs:
            r.join()
        stop.set()
        w.join()
    finally:
        q4.gemv_q4_clear_geometry()
    assert not bad, bad[:3]


def test_block_and_scan_settings_read_whole_beside_a_writer():
    """The block-format and scan settings are single words: readers on other
    threads see either the old or the new setting, never a mix."""
    import threading
    fmt = q4.BLOCK_FORMATS["q4_k"]
    L = q4.lib()
    cfgs = [(1, 4, 2), (2, 8, 0)]
    scans = [(1, 2, 256, 2), (0, 1, 64, 1)]
    stop = threading.Event()
    bad = []

    def writer():
        i = 0
        while not stop.is_set():
            L.gemv_block_set_config(fmt, *cfgs[i % 2])
            L.scan2_set_config(*scans[i % 2])
            i += 1

    def reader():
        for _ in range(5000):
            c = q4.gemv_block_config("q4_k")
            s = q4.scan2_config()
            if tuple(c) not in cfgs or tuple(s) not in scans:
                bad.append((c, s))

    L.gemv_block_set_config(fmt, *cfgs[0])
    L.scan2_set_config(*scans[0])
    try:
        w = threading.Thread(target=writer)
        rs = [threading.Thread(target=reader) for _ in range(3)]
        w.start()
        for r in rs:
            r.start()
        for r in rs:
            r.join()
        stop.set()
        w.join()
    finally:
        L.gemv_block_set_config(fmt, 0, 0, 0)
        L.scan2_set_config(0, 0, 0, 0)
    assert not bad, bad[:3]
