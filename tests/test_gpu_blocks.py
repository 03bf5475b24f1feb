"""GPU parity of the block-format GEMV and dequantiser against the oracle,
through the C ABI.

Bars (per element): dequantised weights bit-exact; GEMVs within
1e-4 * B + 1e-6 of the f64 reference, B the oracle's bound (sum |x| |w|, and
for Q4_K / Q5_K sum |x| (|d s q| + |dmin m|)).  Small and ragged shapes are
compared in full, spanning one to eight passes of 64 units per lane row and
row counts that leave workgroups partly empty; the cera page's shapes and the
4096 x 14336 stream shape are run in the launch configuration the benchmark
times and compared on sampled rows.
"""

import numpy as np
import pytest
import torch

import memory_bandwidth_amd as q4
from oracle import blocks
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
FMTS = list(wl.BLOCK_FORMATS)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run(fmt, x, w):
    y = q4.gemv_block(fmt, to_dev(x), to_dev(w))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def assert_within(y, y_ref, bound, label):
    err = np.abs(y.astype(np.float64) - y_ref)
    tol = blocks.gemv_tolerance(bound)
    bad = ~(err <= tol)
    assert not bad.any(), (f"{label}: {int(bad.sum())}/{bad.size} outputs out of tolerance, "
                           f"worst err/tol {np.nanmax(err / tol):.3g}")


def code(fmt):
    return wl.BLOCK_FORMATS[fmt][0]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(1, 256), (3, 512), (7, 2816), (33, 1024), (5, 4352), (2, 32768)])
def test_dequant_bit_exact(fmt, N, K):
    w = wl.make_block_weights(41, fmt, N, K)
    got = q4.dequant_block(fmt, to_dev(w), K).cpu().numpy()
    want = blocks.dequant(code(fmt), w, K)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), fmt


# K: 4 units (one partly filled pass), 44, exactly 64, 68 (a second pass of
# 4 units), 224 (four passes, the last half full), 512 (the largest K).
SHAPES = [(1, 256), (3, 2816), (17, 4096), (9, 4352), (5, 14336), (2, 32768), (257, 1024)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", SHAPES)
def test_gemv_small_shapes(fmt, N, K):
    w = wl.make_block_weights(42, fmt, N, K)
    x = wl.make_x(43, 1, K)
    y = run(fmt, x, w)
    y_ref, b = blocks.gemv(code(fmt), x, w)
    assert_within(y, y_ref, b, f"{fmt} N={N} K={K}")


@pytest.mark.parametrize("fmt", FMTS)
def test_every_config(fmt):
    """Every (row slots, wavefronts per workgroup) the library runs, with one
    workgroup per row block and with at most one per CU looping over row
    blocks, at 64, 32 and 16 lanes per row (K = 4352 in two passes, 2048,
    1024) and at 65536 x 1024 on sampled rows, where every configuration
    loops."""
    cases = []
    for i, (N, K) in enumerate([(1100, 4352), (1500, 2048), (1030, 1024)]):
        w = wl.make_block_weights(44, fmt, N, K, index=i)
        x = wl.make_x(45, 1, K, index=i)
        cases.append((x, w, None, *blocks.gemv(code(fmt), x, w)))
    w = wl.make_block_weights(44, fmt, 65536, 1024, index=9)
    x = wl.make_x(45, 1, 1024, index=9)
    rows = np.unique(np.r_[0:70, 65536 - 70:65536,
                           np.random.default_rng(56).choice(65536, 64, replace=False)]).astype(np.int64)
    cases.append((x, w, rows, *blocks.gemv(code(fmt), x, w, rows)))
    try:
        for R in ((1, 2) if fmt in ("q5_k", "q6_k") else (1, 2, 4)):
            for W in (4, 8):
                for G in (0, 1):
                    q4.gemv_block_set_config(fmt, R, W, G)
                    assert q4.gemv_block_config(fmt) == (R, W, G)
                    for x, w, rows, y_ref, b in cases:
                        y = run(fmt, x, w)
                        if rows is not None:
                            y = y[:, rows]
                        assert_within(y, y_ref, b, f"{fmt} R={R} W={W} G={G} N={w.shape[0]}")
    finally:
        q4.gemv_block_set_config(fmt, 0, 0, 0)


@pytest.mark.parametrize("fmt", FMTS)
def test_page_and_stream_shapes_sampled(fmt):
    """The cera page's four shapes and the stream shape, sampled rows."""
    shapes = [(n, k) for n, k, _ in wl.BLOCK_SHAPES] + [(14336, 4096)]
    rng = np.random.default_rng(46)
    for i, (N, K) in enumerate(shapes):
        w = wl.make_block_weights(47, fmt, N, K, index=i)
        x = wl.make_x(48, 1, K, index=i)
        y = run(fmt, x, w)
        rows = np.unique(np.r_[0:8, N - 8:N, rng.choice(N, 48, replace=False)]).astype(np.int64)
        y_ref, b = blocks.gemv(code(fmt), x, w, rows)
        assert_within(y[:, rows], y_ref, b, f"{fmt} N={N} K={K}")


def _zero_point_matrix(fmt, N, K):
    """Every weight exactly zero: codes equal to their offsets, K-format
    scales and mins zero."""
    _, e, b, offs = wl.BLOCK_FORMATS[fmt]
    w = wl.make_block_weights(49, fmt, N, K).reshape(N, K // e, b)
    if fmt == "q4_0":
        w[:, :, 2:] = 0x88
    elif fmt == "q8_0":
        w[:, :, 2:] = 0
    elif fmt in ("q4_k", "q5_k"):
        w[:, :, 4:16] = 0
    else:
        w[:, :, 0:128] = 0x00           # low nibbles 0, top bits 2: q = 32
        w[:, :, 128:192] = 0xAA
    return w.reshape(N, -1)


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_point_codes_give_exact_zero(fmt):
    N, K = 19, 4352
    w = _zero_point_matrix(fmt, N, K)
    x = wl.make_x(50, 1, K) * 1e3
    assert not blocks.dequant(code(fmt), w, K).any()
    y = run(fmt, x, w)
    assert np.array_equal(y, np.zeros_like(y)), fmt


@pytest.mark.parametrize("fmt", FMTS)
def test_wide_range_x(fmt):
    N, K = 23, 2816
    w = wl.make_block_weights(51, fmt, N, K)
    x = wl.make_x(52, 1, K) * np.exp2(np.random.default_rng(53).integers(-20, 20, K)).astype(np.float32)
    y = run(fmt, x, w)
    y_ref, b = blocks.gemv(code(fmt), x, w)
    assert_within(y, y_ref, b, fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_non_finite_x_poisons_every_row(fmt):
    N, K = 37, 1024
    w = wl.make_block_weights(58, fmt, N, K)
    for bad in (np.nan, np.inf):
        x = wl.make_x(59, 1, K)
        x[0, 517] = bad
        y = run(fmt, x, w)
        assert not np.isfinite(y).any(), (fmt, bad)


@pytest.mark.parametrize("fmt", FMTS)
def test_nan_scale_poisons_only_its_row(fmt):
    N, K = 9, 1024
    _, e, bb, offs = wl.BLOCK_FORMATS[fmt]
    w = wl.make_block_weights(54, fmt, N, K).reshape(N, K // e, bb)
    w[4, 1, offs[0]:offs[0] + 2] = [0x00, 0x7E]          # binary16 NaN as the scale d
    w = w.reshape(N, -1)
    x = wl.make_x(55, 1, K)
    y = run(fmt, x, w)
    assert np.isnan(y[0, 4])
    ok = np.arange(N) != 4
    y_ref, b = blocks.gemv(code(fmt), x, w, np.nonzero(ok)[0])
    assert_within(y[:, ok], y_ref, b, fmt)


def test_zero_rows_and_validation():
    x = torch.zeros((1, 256), device=DEV)
    y = torch.empty((1, 0), device=DEV)
    q4.gemv_block("q4_0", x, torch.empty((0, 144), dtype=torch.uint8, device=DEV), out=y)
    with pytest.raises(q4.Q4Error):
        q4.gemv_block("q4_0", torch.zeros((2, 256), device=DEV),
                      torch.zeros((3, 144), dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError):
        q4.gemv_block("q4_k", x, torch.zeros((3, 145), dtype=torch.uint8, device=DEV))
