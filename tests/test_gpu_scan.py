"""GPU parity of the 2-bit corpus scan against its oracle, through the C ABI.

Bar: |score - score_ref| <= 1e-4 * sum_d |lut term| + 1e-6 per output, and
bit-exact on integer tables (every partial sum an exact fp32 integer).
Shapes span one to sixteen 64-dimension chunks, 1 to 8 queries (one or two
groups of four, partly filled), vector counts that leave workgroups partly
empty, every configuration of the page's knobs, and the page's 65,536 x 8
workload (D = 768) on sampled vectors.
"""

import numpy as np
import pytest
import torch

import memory_bandwidth_amd as q4
from oracle import scan
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def run(codes, lut):
    s = q4.scan2(torch.from_numpy(codes.view(np.int32)).to(DEV), torch.from_numpy(lut).to(DEV))
    torch.cuda.synchronize()
    return s.cpu().numpy()


def assert_within(s, ref, bound, label):
    err = np.abs(s.astype(np.float64) - ref)
    tol = scan.scan_tolerance(bound)
    bad = ~(err <= tol)
    assert not bad.any(), (f"{label}: {int(bad.sum())}/{bad.size} out of tolerance, worst err/tol "
                           f"{np.nanmax(err / tol):.3g}")


@pytest.mark.parametrize("V,D,Q", [(1, 64, 1), (1, 64, 8), (3, 128, 6), (257, 128, 3), (1000, 768, 8),
                                   (333, 1024, 5), (64, 192, 4), (4097, 256, 8)])
def test_scan_small(V, D, Q):
    codes = wl.make_scan_codes(61, V, D)
    lut = wl.make_scan_lut(61, Q, D)
    ref, b = scan.scan(codes, lut)
    assert_within(run(codes, lut), ref, b, f"V={V} D={D} Q={Q}")


def test_every_config():
    cases = []
    # D = 768: 12 chunks (8 threads per vector fall back to 4); D = 512: 8
    # chunks; D = 320: 5 chunks (one thread per vector).
    for i, (V, D, Q) in enumerate([(3000, 768, 8), (2100, 512, 6), (1500, 320, 3)]):
        codes = wl.make_scan_codes(62, V, D, index=i)
        lut = wl.make_scan_lut(62, Q, D, index=i)
        cases.append((codes, lut, *scan.scan(codes, lut)))
    try:
        for lds in (1, 0):
            for vpt in (1, 2):
                for tpg in (64, 256, 1024):
                    for tpv in (0, 1, 2, 4, 8):
                        q4.scan2_set_config(lds, vpt, tpg, tpv)
                        assert q4.scan2_config() == (lds, vpt, tpg, tpv)
                        for codes, lut, ref, b in cases:
                            assert_within(run(codes, lut), ref, b,
                                          f"lds={lds} vpt={vpt} tpg={tpg} tpv={tpv} D={lut.shape[1]}")
    finally:
        q4.scan2_set_config(0, 0, 0, 0)


def test_table_in_memory_long_vectors():
    """D = 4096 (beyond the LDS table limit) with the table read from memory."""
    codes = wl.make_scan_codes(63, 700, 4096)
    lut = wl.make_scan_lut(63, 8, 4096)
    ref, b = scan.scan(codes, lut)
    try:
        q4.scan2_set_config(0, 1, 256, 4)
        assert_within(run(codes, lut), ref, b, "D=4096")
    finally:
        q4.scan2_set_config(0, 0, 0, 0)
    with pytest.raises(q4.Q4Error):
        run(codes, lut)                       # the default (LDS table) refuses D > 1024


def test_integer_table_is_exact():
    rng = np.random.default_rng(64)
    V, D, Q = 2000, 768, 8
    c = rng.integers(0, 4, (V, D)).astype(np.uint64)
    codes = (c.reshape(V, D // 16, 16) << (2 * np.arange(16, dtype=np.uint64))).sum(axis=2).astype(np.uint32)
    lut = rng.integers(-50, 51, (Q, D, 4)).astype(np.float32)
    ref, _ = scan.scan(codes, lut)
    assert np.array_equal(run(codes, lut).astype(np.float64), ref)


@pytest.mark.parametrize("V,D,Q,cfg", [(40000, 768, 8, (1, 1, 64, 1)), (40000, 768, 3, (1, 1, 64, 1)),
                                       (150001, 128, 8, (1, 2, 256, 1)), (70000, 320, 5, (0, 1, 256, 1))])
def test_workgroups_loop_over_vector_blocks(V, D, Q, cfg):
    """More vector blocks than workgroups that fit the chip at once: each
    workgroup builds its table once and scans several blocks."""
    codes = wl.make_scan_codes(67, V, D)
    lut = wl.make_scan_lut(67, Q, D)
    rows = np.unique(np.r_[0:300, V - 300:V, np.random.default_rng(68).choice(V, 2000, replace=False)])
    ref, b = scan.scan(codes, lut, rows)
    try:
        q4.scan2_set_config(*cfg)
        assert_within(run(codes, lut)[rows], ref, b, f"V={V} D={D} Q={Q} cfg={cfg}")
    finally:
        q4.scan2_set_config(0, 0, 0, 0)


def test_page_workload_sampled():
    V, Q, D = wl.SCAN_VECTORS, wl.SCAN_QUERIES, wl.SCAN_DIM
    codes = wl.make_scan_codes(65, V, D)
    lut = wl.make_scan_lut(65, Q, D)
    s = run(codes, lut)
    rows = np.unique(np.r_[0:64, V - 64:V, np.random.default_rng(66).choice(V, 256, replace=False)])
    ref, b = scan.scan(codes, lut, rows)
    assert_within(s[rows], ref, b, "65536 x 8, D = 768")
