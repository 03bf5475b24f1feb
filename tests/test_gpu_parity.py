"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Bars (all per element):
  * codes and dequantised weights: bit-exact;
  * GEMVs on integer-exact inputs: bit-exact;
  * GEMVs otherwise: |y - y_ref| <= 1e-4 * sum|w x| + 1e-6, y_ref in f64.
Small and ragged shapes are compared in full; the configured full-size
shapes are run in the launch configuration the benchmark times and compared
on sampled rows the oracle computes one by one.
"""

import os

import numpy as np
import pytest
import torch

import memory_bandwidth_amd as q4
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def dev(d):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for k, v in d.items()}


def run_q4(t, g, M=None):
    y = q4.gemv_q4(t["x"], t["wq"], t["scales"], t["zeros"], g)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def assert_within(y, y_ref, bound, label):
    err = np.abs(y.astype(np.float64) - y_ref)
    tol = oracle.gemv_tolerance(bound)
    bad = err > tol
    assert not bad.any(), (f"{label}: {int(bad.sum())}/{bad.size} outputs out of tolerance, "
                           f"worst err/tol {np.max(err / tol):.3g}")


def sample_rows(N, n, seed):
    rng = np.random.default_rng(seed)
    edge = np.r_[0:min(N, 40), max(0, N - 40):N]
    mid = rng.choice(N, size=min(N, n), replace=False)
    return np.unique(np.r_[edge, mid]).astype(np.int64)


# ---------------------------------------------------------------- workloads

def test_single_896():
    s = wl.SMALL_896
    d = wl.make_q4_problem(wl.workload_seed(0), s)
    y = run_q4(dev(d), s.g)
    y_ref, b = oracle.gemv_q4(d["x"], d["wq"], d["scales"], d["zeros"], s.g)
    assert_within(y, y_ref, b, s.label)


def test_fused_decoder_layer():
    """The decoder layer in four launches: q, k and v as one matrix whose rows
    are theirs one after another, o, the SwiGLU block of gate and up, down."""
    mats = [wl.make_q4_weights(wl.workload_seed(1), s.N, s.K, s.g, s.s_lo, s.s_hi, index=10 + i)
            for i, s in enumerate(wl.DECODER_LAYER)]
    x = wl.make_x(wl.workload_seed(1), 1, 896, index=10)
    qkv = wl.fuse_rows(*mats[:3])
    assert qkv["wq"].shape == (896 + 128 + 128, 448)
    t = dev(dict(qkv, x=x))
    y = run_q4(t, 32)
    y_ref, b = oracle.gemv_q4(x, qkv["wq"], qkv["scales"], qkv["zeros"], 32)
    assert_within(y, y_ref, b, "fused qkv")
    o = 0
    for i in range(3):                         # each slice is that matrix's GEMV
        m = mats[i]
        yi, bi = oracle.gemv_q4(x, m["wq"], m["scales"], m["zeros"], 32)
        assert_within(y[:, o:o + m["wq"].shape[0]], yi, bi, wl.DECODER_LAYER[i].label)
        o += m["wq"].shape[0]
    gate, up = dev(mats[4]), dev(mats[5])
    ys = q4.gemv_q4_swiglu(t["x"], (gate["wq"], gate["scales"], gate["zeros"]),
                           (up["wq"], up["scales"], up["zeros"]), 32)
    torch.cuda.synchronize()
    ys_ref, tol = oracle.swiglu(x, (mats[4]["wq"], mats[4]["scales"], mats[4]["zeros"]),
                                (mats[5]["wq"], mats[5]["scales"], mats[5]["zeros"]), 32)
    assert np.all(np.abs(ys.cpu().numpy().astype(np.float64) - ys_ref) <= tol)


def test_decoder_layer():
    for i, s in enumerate(wl.DECODER_LAYER):
        d = wl.make_q4_problem(wl.workload_seed(1), s, index=i)
        t = dev(d)
        y = run_q4(t, s.g)
        y_ref, b = oracle.gemv_q4(d["x"], d["wq"], d["scales"], d["zeros"], s.g)
        assert_within(y, y_ref, b, s.label)
        # the same shape as the dense fp32 control, on the exact dequantised weights
        w, _ = oracle.dequant(d["wq"], d["scales"], d["zeros"], s.K, s.g)
        yf = q4.gemv_f32(t["x"], torch.from_numpy(w).to(DEV))
        torch.cuda.synchronize()
        yf_ref, bf = oracle.gemv_f32(d["x"], w)
        assert_within(yf.cpu().numpy(), yf_ref, bf, "f32 " + s.label)


def test_lm_head_sampled():
    s = wl.LM_HEAD
    d = wl.make_q4_problem(wl.workload_seed(2), s)
    y = run_q4(dev(d), s.g)
    rows = sample_rows(s.N, 3000, 2)
    y_ref, b = oracle.gemv_q4(d["x"], d["wq"], d["scales"], d["zeros"], s.g, rows=rows)
    assert_within(y[:, rows], y_ref, b, s.label)


@pytest.mark.parametrize("M", [1, 4, 8])
def test_ffn_sampled(M):
    for i, s in enumerate(wl.ffn_8b(M)):
        d = wl.make_q4_problem(wl.workload_seed(3), s, index=i)
        y = run_q4(dev(d), s.g)
        rows = sample_rows(s.N, 200, 3 + M)
        y_ref, b = oracle.gemv_q4(d["x"], d["wq"], d["scales"], d["zeros"], s.g, rows=rows)
        assert_within(y[:, rows], y_ref, b, s.label)


def test_stream_sampled():
    s = wl.STREAM_SHAPE
    seed = wl.workload_seed(4)
    x = wl.make_x(seed, 1, s.K)
    xt = torch.from_numpy(x).to(DEV)
    for idx in (0, 13, 31):
        d = wl.make_q4_weights(seed, s.N, s.K, s.g, s.s_lo, s.s_hi, index=idx)
        t = dev(d)
        y = q4.gemv_q4(xt, t["wq"], t["scales"], t["zeros"], s.g)
        torch.cuda.synchronize()
        rows = sample_rows(s.N, 300, idx)
        y_ref, b = oracle.gemv_q4(x, d["wq"], d["scales"], d["zeros"], s.g, rows=rows)
        assert_within(y.cpu().numpy()[:, rows], y_ref, b, f"{s.label} matrix {idx}")
    # dense control on the same shape, weights dequantised by the oracle
    w, _ = oracle.dequant(d["wq"], d["scales"], d["zeros"], s.K, s.g)
    yf = q4.gemv_f32(xt, torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    yf_ref, bf = oracle.gemv_f32(x, w, rows=rows)
    assert_within(yf.cpu().numpy()[:, rows], yf_ref, bf, "f32 control " + s.label)


# ---------------------------------------------------------------- ragged / edge shapes

RAGGED = [
    # M, N, K, g
    (1, 1, 32, 32), (1, 3, 64, 32), (2, 5, 96, 32), (1, 7, 128, 128), (3, 17, 256, 128),
    (1, 31, 512, 32), (4, 33, 544, 32), (1, 63, 1024, 32), (5, 64, 1056, 32), (1, 65, 2048, 128),
    (8, 67, 2080, 32), (1, 127, 4096, 128), (6, 129, 4224, 128), (1, 1000, 896, 32),
    (7, 257, 4864, 32), (8, 67, 14336, 128), (1, 45, 14336, 128), (2, 300, 8192, 128),
    (1, 1, 16384, 128), (8, 9, 18432, 128), (1, 4097, 384, 128), (8, 1, 32, 32),
    (8, 100, 32768, 128), (3, 70, 32768, 32), (1, 33, 32768, 128),
    # the longest rows the one-row integer kernel takes: all of x's records fill the LDS
    (1, 4096, 19232, 32), (1, 2, 19264, 32),
    # several x segments of the multiply-add kernel, the last one shorter
    (3, 300, 14336, 128), (5, 200, 14336, 128), (4, 96, 14336, 32), (6, 50, 9216, 128),
]


@pytest.mark.parametrize("M,N,K,g", RAGGED, ids=[f"M{a}N{b}K{c}g{d}" for a, b, c, d in RAGGED])
def test_gemv_q4_ragged(M, N, K, g):
    s = wl.Q4Shape(M, N, K, g, 0.002, 0.02)
    d = wl.make_q4_problem(1000 + N, s)
    y = run_q4(dev(d), g)
    y_ref, b = oracle.gemv_q4(d["x"], d["wq"], d["scales"], d["zeros"], g)
    assert_within(y, y_ref, b, f"M{M} N{N} K{K} g{g}")


LONGEST = [(1, 3, 1 << 24, 128), (8, 2, 1 << 24, 32), (3, 5, (1 << 24) - 128, 128)]


@pytest.mark.parametrize("M,N,K,g", LONGEST, ids=[f"M{a}N{b}K{c}g{d}" for a, b, c, d in LONGEST])
def test_gemv_q4_longest_k(M, N, K, g):
    """The longest K a call accepts (2^24): every 32-bit buffer offset of the
    kernels is then at its largest.  With and without a workspace (a K split
    over workgroups where the plan makes one)."""
    print(f"longest K: M{M} N{N} K{K} g{g}", flush=True)
    s = wl.Q4Shape(M, N, K, g, 0.002, 0.02)
    d = wl.make_q4_problem(4242 + M, s)
    t = dev(d)
    y_ref, b = oracle.gemv_q4(d["x"], d["wq"], d["scales"], d["zeros"], g)
    y = q4.gemv_q4(t["x"], t["wq"], t["scales"], t["zeros"], g)
    y_plain = q4.gemv_q4(t["x"], t["wq"], t["scales"], t["zeros"], g, workspace=False)
    torch.cuda.synchronize()
    assert_within(y.cpu().numpy(), y_ref, b, f"longest K M{M} N{N} K{K} g{g}")
    assert_within(y_plain.cpu().numpy(), y_ref, b, f"longest K, no workspace, M{M} N{N} K{K} g{g}")


EXACT = [(1, 14336, 4096, 128), (1, 4096, 14336, 128), (8, 333, 14336, 128), (4, 515, 4096, 128),
         (1, 896, 896, 32), (3, 2000, 4864, 32), (8, 77, 640, 32), (2, 1024, 32768, 128)]


@pytest.mark.parametrize("M,N,K,g", EXACT, ids=[f"M{a}N{b}K{c}g{d}" for a, b, c, d in EXACT])
def test_gemv_q4_integer_exact(M, N, K, g):
    d = wl.make_exact_problem(77 + M, M, N, K, g)
    y = run_q4(dev(d), g)
    y_ref, _ = oracle.gemv_q4(d["x"], d["wq"], d["scales"], d["zeros"], g)
    assert np.array_equal(y.astype(np.float64), y_ref), np.max(np.abs(y - y_ref))


def test_gemv_q4_q_equals_z_is_exactly_zero():
    M, N, K, g = 4, 300, 4096, 128
    d = wl.make_q4_problem(5, wl.Q4Shape(M, N, K, g, 0.002, 0.01))
    z = np.stack([d["zeros"] & 15, d["zeros"] >> 4], -1).reshape(N, -1)[:, :K // g]
    codes = np.repeat(z, g, axis=1).astype(np.uint8)
    d["wq"] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    y = run_q4(dev(d), g)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("N,K", [(300, 4096), (77, 14336), (5, 2048)])
def test_gemv_q4_integer_path_q_equals_z_is_exactly_zero(N, K):
    """One activation row takes the integer path; q == z must still give exactly 0."""
    g = 128
    assert q4.gemv_q4_path(1, N, K, g) == q4.Q4_PATH_INTEGER
    d = wl.make_q4_problem(6, wl.Q4Shape(1, N, K, g, 0.002, 0.01))
    z = np.stack([d["zeros"] & 15, d["zeros"] >> 4], -1).reshape(N, -1)[:, :K // g]
    codes = np.repeat(z, g, axis=1).astype(np.uint8)
    d["wq"] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    y = run_q4(dev(d), g)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("M,N,K", [(1, 257, 4096), (1, 96, 14336), (1, 33, 1056), (4, 129, 4096),
                                   (8, 40, 14336)])
def test_gemv_q4_wide_dynamic_range_x(M, N, K):
    """x magnitudes spread over ten decades inside every 32-value chunk (the
    integer path rounds each chunk to 23 bits of its largest |x|)."""
    g = 128 if K % 128 == 0 else 32
    d = wl.make_q4_problem(12, wl.Q4Shape(M, N, K, g, 0.002, 0.02))
    rng = np.random.default_rng(12)
    d["x"] = (d["x"] * 10.0 ** rng.uniform(-6, 4, size=d["x"].shape)).astype(np.float32)
    y = run_q4(dev(d), g)
    y_ref, b = oracle.gemv_q4(d["x"], d["wq"], d["scales"], d["zeros"], g)
    assert_within(y, y_ref, b, f"wide-range x M{M} N{N} K{K}")


def _large_x_meets_zero_point(d, M, N, K, g, seed, big_exp=14, small=(0.5, 1.0)):
    """In every 32-value chunk of every x row the first value is 2^big_exp and
    meets q == z (so it carries no weight), while the other 31 values are
    2^big_exp / small times smaller and meet random codes: only the small
    values carry weight, and the plain bound is set by them alone."""
    rng = np.random.default_rng(seed)
    x = rng.uniform(*small, size=(M, K)) * rng.choice([-1.0, 1.0], size=(M, K))
    x[:, 0::32] = 2.0 ** big_exp
    d["x"] = x.astype(np.float32)
    codes = np.stack([d["wq"] & 15, d["wq"] >> 4], -1).reshape(N, K)
    z = np.stack([d["zeros"] & 15, d["zeros"] >> 4], -1).reshape(N, -1)[:, :K // g]
    codes[:, 0::32] = np.repeat(z, g // 32, axis=1)
    d["wq"] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return d


X_RANGE = [(1, 129, 4096, 128), (1, 40, 2048, 128), (1, 300, 896, 32), (1, 77, 14336, 128),
           (1, 5000, 1024, 32), (2, 300, 8192, 128), (4, 129, 4096, 128), (8, 67, 4096, 128),
           (8, 40, 14336, 128), (3, 33, 1056, 32), (5, 64, 32768, 128)]


@pytest.mark.parametrize("M,N,K,g", X_RANGE, ids=[f"M{a}N{b}K{c}g{d}" for a, b, c, d in X_RANGE])
def test_gemv_q4_small_x_beside_large_at_plain_bound(M, N, K, g):
    """Every chunk's large x meets q == z and only values 2^14-2^15 times
    smaller carry weight; each output within the plain bound
    |y - y_ref| <= 1e-4 * sum|w x| + 1e-6, on every path: one row (64 and 32
    lanes per row, K-split), 2-8 rows (one and several x segments), the
    multiply-add path (M = 3, K = 1056)."""
    d = wl.make_q4_problem(14 + M, wl.Q4Shape(M, N, K, g, 0.002, 0.01))
    d = _large_x_meets_zero_point(d, M, N, K, g, 14 + M)
    y = run_q4(dev(d), g)
    y_ref, b = oracle.gemv_q4(d["x"], d["wq"], d["scales"], d["zeros"], g)
    assert_within(y, y_ref, b, f"large x on q == z, M{M} N{N} K{K} path {q4.gemv_q4_path(M, N, K, g)}")


@pytest.mark.parametrize("M,N,K", [(1, 96, 4096), (4, 129, 4096), (8, 48, 4096), (8, 40, 14336), (2, 70, 8192)])
def test_gemv_q4_every_small_x_corrected(M, N, K):
    """Chunks whose 31 small values all take the fp32 residual correction
    (2^20 beside values near 1): with 2 to 8 rows more half chunks hold
    flagged values than the residual pool has slots, so the rest are
    recomputed from x.  Plain bound."""
    g = 128
    d = wl.make_q4_problem(15 + M, wl.Q4Shape(M, N, K, g, 0.002, 0.01))
    d = _large_x_meets_zero_point(d, M, N, K, g, 15 + M, big_exp=20)
    y = run_q4(dev(d), g)
    y_ref, b = oracle.gemv_q4(d["x"], d["wq"], d["scales"], d["zeros"], g)
    assert_within(y, y_ref, b, f"all small x corrected, M{M} N{N} K{K}")


@pytest.mark.parametrize("M,N,K,g", [(1, 300, 4096, 128), (1, 4864, 896, 32), (4, 129, 4096, 128),
                                     (1, 70, 14336, 128)])
def test_gemv_q4_swiglu_small_x_beside_large(M, N, K, g):
    """The q == z construction through both projections of the SwiGLU block
    (one launch at one row on the integer path, else two)."""
    s = wl.Q4Shape(M, N, K, g, 0.002, 0.01)
    dg = _large_x_meets_zero_point(wl.make_q4_problem(320 + N, s, index=0), M, N, K, g, 320 + N)
    du = wl.make_q4_problem(320 + N, s, index=1)
    du["x"] = dg["x"]
    codes_g = np.stack([dg["wq"] & 15, dg["wq"] >> 4], -1).reshape(N, K)
    zu = np.stack([du["zeros"] & 15, du["zeros"] >> 4], -1).reshape(N, -1)[:, :K // g]
    cu = np.stack([du["wq"] & 15, du["wq"] >> 4], -1).reshape(N, K)
    cu[:, 0::32] = np.repeat(zu, g // 32, axis=1)
    du["wq"] = (cu[:, 0::2] | (cu[:, 1::2] << 4)).astype(np.uint8)
    assert codes_g.shape == cu.shape
    tg, tu = dev(dg), dev(du)
    y = q4.gemv_q4_swiglu(tg["x"], (tg["wq"], tg["scales"], tg["zeros"]),
                          (tu["wq"], tu["scales"], tu["zeros"]), g)
    torch.cuda.synchronize()
    y_ref, tol = oracle.swiglu(dg["x"], (dg["wq"], dg["scales"], dg["zeros"]),
                               (du["wq"], du["scales"], du["zeros"]), g)
    err = np.abs(y.cpu().numpy().astype(np.float64) - y_ref)
    assert np.all(err <= tol), f"{int((err > tol).sum())} outputs out of tolerance, worst {np.max(err / tol):.3g}"


@pytest.mark.parametrize("M,K", [(1, 4096), (1, 896), (3, 4096)])
def test_gemv_q4_nan_in_x_propagates(M, K):
    N, g = 64, 128
    d = wl.make_q4_problem(13, wl.Q4Shape(M, N, K, g, 0.002, 0.02))
    d["x"][:, 77] = np.nan
    y = run_q4(dev(d), g)
    assert np.isnan(y).all()


def test_stream_shape_takes_integer_path():
    s = wl.STREAM_SHAPE
    assert q4.gemv_q4_path(s.M, s.N, s.K, s.g) == q4.Q4_PATH_INTEGER


def test_gemv_q4_linearity_and_rows():
    """Doubling x doubles y exactly; row m of an M=8 call matches M=1 on x[m]."""
    s = wl.Q4Shape(8, 1234, 4096, 128, 0.002, 0.01)
    d = wl.make_q4_problem(9, s)
    t = dev(d)
    y = run_q4(t, s.g)
    t2 = dict(t, x=t["x"] * 2)
    y2 = run_q4(t2, s.g)
    assert np.array_equal(y2, 2 * y)
    y_ref, b = oracle.gemv_q4(d["x"], d["wq"], d["scales"], d["zeros"], s.g)
    for m in (0, 5, 7):
        t1 = dict(t, x=t["x"][m:m + 1].contiguous())
        assert_within(run_q4(t1, s.g), y_ref[m:m + 1], b[m:m + 1], f"row {m} as M=1")


def test_gemv_q4_deterministic_and_guarded():
    s = wl.Q4Shape(2, 1001, 4096, 128, 0.002, 0.01)
    d = wl.make_q4_problem(10, s)
    t = dev(d)
    buf = torch.full((s.M * s.N + 4096,), float("nan"), device=DEV)
    out = buf[: s.M * s.N].view(s.M, s.N)
    q4.gemv_q4(t["x"], t["wq"], t["scales"], t["zeros"], s.g, out=out)
    a = out.clone()
    q4.gemv_q4(t["x"], t["wq"], t["scales"], t["zeros"], s.g, out=out)
    torch.cuda.synchronize()
    assert torch.equal(a, out)
    assert torch.isnan(buf[s.M * s.N:]).all(), "write past the end of y"


def test_gemv_q4_empty_n():
    x = torch.zeros((1, 128), device=DEV)
    wq = torch.zeros((0, 64), dtype=torch.uint8, device=DEV)
    sc = torch.zeros((0, 4), dtype=torch.float16, device=DEV)
    zp = torch.zeros((0, 2), dtype=torch.uint8, device=DEV)
    y = q4.gemv_q4(x, wq, sc, zp, 32)
    assert y.shape == (1, 0)


def test_gemv_q4_graph_replay():
    s = wl.STREAM_SHAPE
    d = wl.make_q4_problem(11, s)
    t = dev(d)
    eager = q4.gemv_q4(t["x"], t["wq"], t["scales"], t["zeros"], s.g)
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            q4.gemv_q4(t["x"], t["wq"], t["scales"], t["zeros"], s.g, out=out)
    for i in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"


# ---------------------------------------------------------------- dequant_q4

DQ = [(1, 32, 32), (3, 96, 32), (17, 256, 128), (64, 896, 32), (1000, 4096, 128), (7, 4864, 32)]


@pytest.mark.parametrize("N,K,g", DQ, ids=[f"N{a}K{b}g{c}" for a, b, c in DQ])
def test_dequant_bit_exact(N, K, g):
    d = wl.make_q4_weights(20 + N, N, K, g, 0.002, 0.02)
    t = dev(d)
    w, c = q4.dequant_q4(t["wq"], t["scales"], t["zeros"], g)
    torch.cuda.synchronize()
    w_ref, c_ref = oracle.dequant(d["wq"], d["scales"], d["zeros"], K, g)
    assert np.array_equal(c.cpu().numpy(), c_ref)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), w_ref.view(np.uint32))


def test_dequant_special_scales():
    """Subnormal, negative, huge and zero binary16 scales; NaN/Inf where the math gives them."""
    N, K, g = 64, 256, 32
    d = wl.make_q4_weights(30, N, K, g, 0.01, 0.02)
    rng = np.random.default_rng(30)
    specials = np.array([0x0001, 0x03FF, 0x0400, 0x8001, 0xBC00, 0x7BFF, 0xFBFF, 0x0000,
                         0x8000, 0x7C00, 0xFC00, 0x7E00], np.uint16)
    d["scales"] = rng.choice(specials, size=d["scales"].shape).astype(np.uint16)
    t = dev(d)
    w, c = q4.dequant_q4(t["wq"], t["scales"], t["zeros"], g)
    torch.cuda.synchronize()
    w_ref, c_ref = oracle.dequant(d["wq"], d["scales"], d["zeros"], K, g)
    w = w.cpu().numpy()
    nan = np.isnan(w_ref)
    assert np.array_equal(np.isnan(w), nan)
    assert np.array_equal(w[~nan].view(np.uint32), w_ref[~nan].view(np.uint32))
    assert np.array_equal(c.cpu().numpy(), c_ref)


def test_dequant_codes_only_and_weights_only():
    N, K, g = 50, 512, 128
    d = wl.make_q4_weights(31, N, K, g, 0.002, 0.01)
    t = dev(d)
    w, c = q4.dequant_q4(t["wq"], t["scales"], t["zeros"], g, want_weights=False)
    assert w is None
    w2, c2 = q4.dequant_q4(t["wq"], t["scales"], t["zeros"], g, want_codes=False)
    torch.cuda.synchronize()
    w_ref, c_ref = oracle.dequant(d["wq"], d["scales"], d["zeros"], K, g)
    assert c2 is None and np.array_equal(c.cpu().numpy(), c_ref)
    assert np.array_equal(w2.cpu().numpy().view(np.uint32), w_ref.view(np.uint32))


# ---------------------------------------------------------------- gemv_f32

# (2, 9000, 4096) and (1, 4097, 4096): K splits chosen to spread the workgroups evenly
F32 = [(1, 1, 4), (1, 33, 60), (2, 65, 128), (1, 1000, 896), (8, 129, 4096), (3, 77, 16400),
       (1, 4097, 4096), (5, 31, 20000), (2, 9000, 4096)]


@pytest.mark.parametrize("M,N,K", F32, ids=[f"M{a}N{b}K{c}" for a, b, c in F32])
def test_gemv_f32(M, N, K):
    rng = np.random.default_rng(M * 1000 + N)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    y = q4.gemv_f32(torch.from_numpy(x).to(DEV), torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    y_ref, b = oracle.gemv_f32(x, w)
    assert_within(y.cpu().numpy(), y_ref, b, f"f32 M{M} N{N} K{K}")


def test_gemv_f32_integer_exact():
    rng = np.random.default_rng(3)
    x = rng.integers(-3, 4, size=(2, 4096)).astype(np.float32)
    w = rng.integers(-64, 65, size=(515, 4096)).astype(np.float32)
    y = q4.gemv_f32(torch.from_numpy(x).to(DEV), torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    y_ref, _ = oracle.gemv_f32(x, w)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y_ref)


# ---------------------------------------------------------------- probes

@pytest.mark.parametrize("n,parts", [(0, 3), (4, 1), (1 << 20, 7), ((1 << 24) + 36, 2048)])
def test_read_reduce_ones(n, parts):
    buf = torch.ones(n, device=DEV)
    p = q4.read_reduce(buf, parts)
    torch.cuda.synchronize()
    assert float(p.double().sum()) == float(n)


def test_read_reduce_random():
    host = wl.make_probe_buffer(3 * (1 << 22) + 12) - np.float32(0.5)
    p = q4.read_reduce(torch.from_numpy(host).to(DEV), 1024)
    torch.cuda.synchronize()
    s, a = oracle.buffer_sum(host)
    assert abs(float(p.double().sum()) - s) <= 1e-5 * a + 1e-6


@pytest.mark.parametrize("n,parts,passes", [(0, 3, 2), (4, 1, 3), (1 << 20, 7, 5), ((1 << 22) + 36, 2048, 16)])
def test_read_reduce_passes_ones(n, parts, passes):
    buf = torch.ones(n, device=DEV)
    p = q4.read_reduce_passes(buf, parts, passes)
    torch.cuda.synchronize()
    assert float(p.double().sum()) == float(n * passes)


@pytest.mark.parametrize("n,blocks,passes", [(4, 0, 1), (4096, 3, 2), ((1 << 22) + 8, 0, 1),
                                             ((1 << 22) + 8, 65536, 3), ((1 << 20) + 4, 1, 1)])
def test_copy_vec4(n, blocks, passes):
    src = torch.from_numpy(wl.make_probe_buffer(n)).to(DEV)
    buf = torch.full((n + 64,), float("nan"), device=DEV)
    q4.copy_vec4(src, buf[:n], passes=passes, n_blocks=blocks)
    torch.cuda.synchronize()
    assert torch.equal(buf[:n], src)
    assert bool(torch.isnan(buf[n:]).all())


@pytest.mark.parametrize("n,blocks", [(4, 0), (4096, 3), ((1 << 22) + 8, 0), ((1 << 22) + 8, 65536)])
def test_write_fill(n, blocks):
    buf = torch.full((n + 64,), float("nan"), device=DEV)
    q4.write_fill(buf[:n], -1.5, blocks)
    torch.cuda.synchronize()
    assert bool((buf[:n] == -1.5).all())
    assert bool(torch.isnan(buf[n:]).all())


# ---------------------------------------------------------------- SwiGLU block

SWIGLU = [(1, 14336, 4096, 128), (1, 4864, 896, 32), (4, 515, 4096, 128), (8, 67, 14336, 128),
          (3, 17, 256, 128), (2, 300, 8192, 128), (5, 129, 4224, 128)]


@pytest.mark.parametrize("M,N,K,g", SWIGLU, ids=[f"M{a}N{b}K{c}g{d}" for a, b, c, d in SWIGLU])
def test_gemv_q4_swiglu(M, N, K, g):
    s = wl.Q4Shape(M, N, K, g, 0.002, 0.02)
    dg = wl.make_q4_problem(300 + N, s, index=0)
    du = wl.make_q4_problem(300 + N, s, index=1)
    tg, tu = dev(dg), dev(du)
    y = q4.gemv_q4_swiglu(tg["x"], (tg["wq"], tg["scales"], tg["zeros"]),
                          (tu["wq"], tu["scales"], tu["zeros"]), g)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    rows = sample_rows(N, 400, N) if N > 2000 else None
    y_ref, tol = oracle.swiglu(dg["x"], (dg["wq"], dg["scales"], dg["zeros"]),
                               (du["wq"], du["scales"], du["zeros"]), g, rows=rows)
    if rows is not None:
        y = y[:, rows]
    bad = np.abs(y - y_ref) > tol
    assert not bad.any(), f"{int(bad.sum())}/{bad.size} outputs out of tolerance"


@pytest.mark.parametrize("M,N,K", [(1, 4864, 896), (1, 300, 4096), (4, 129, 4096)])
def test_gemv_q4_swiglu_nan_in_x_poisons_its_row(M, N, K):
    g = 32 if K % 128 else 128
    s = wl.Q4Shape(M, N, K, g, 0.002, 0.02)
    dg = wl.make_q4_problem(310 + N, s, index=0)
    du = wl.make_q4_problem(310 + N, s, index=1)
    x = dg["x"].copy()
    x[M - 1, K // 3] = np.nan
    tg, tu = dev(dict(dg, x=x)), dev(du)
    y = q4.gemv_q4_swiglu(tg["x"], (tg["wq"], tg["scales"], tg["zeros"]),
                          (tu["wq"], tu["scales"], tu["zeros"]), g)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert np.isnan(y[M - 1]).all()
    assert np.isfinite(y[:M - 1]).all()


def test_gemv_q4_swiglu_zero_gate_is_exactly_zero():
    M, N, K, g = 1, 96, 4096, 128
    s = wl.Q4Shape(M, N, K, g, 0.002, 0.02)
    d = wl.make_q4_problem(31, s)
    z = np.stack([d["zeros"] & 15, d["zeros"] >> 4], -1).reshape(N, -1)[:, :K // g]
    codes = np.repeat(z, g, axis=1).astype(np.uint8)
    gate = dict(d, wq=(codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8))
    t, tg = dev(d), dev(gate)
    y = q4.gemv_q4_swiglu(t["x"], (tg["wq"], tg["scales"], tg["zeros"]),
                          (t["wq"], t["scales"], t["zeros"]), g)
    torch.cuda.synchronize()
    assert np.all(y.cpu().numpy() == 0.0)


# ---------------------------------------------------------------- K split over workgroups (gemv_q4_ws)

WS_SHAPES = [
    # M, N, K, g: several x segments unsplit, so gemv_q4_ws splits K over workgroups
    (8, 4096, 14336, 128), (4, 4096, 14336, 128), (3, 300, 14336, 128), (8, 100, 32768, 128),
    (5, 77, 9216, 32), (8, 2048, 28672, 128), (6, 33, 14336, 128), (7, 1, 16384, 32),
]


@pytest.mark.parametrize("M,N,K,g", WS_SHAPES, ids=[f"M{a}N{b}K{c}g{d}" for a, b, c, d in WS_SHAPES])
def test_gemv_q4_workspace_split(M, N, K, g):
    """gemv_q4_ws with its workspace (partial sums of a K split, then their
    sum) and gemv_q4 without one both meet the bound; a workspace one byte
    short runs gemv_q4's plan."""
    n = q4.gemv_q4_workspace_size(M, N, K, g)
    assert n > 0 and n % (4 * M * N) == 0 and 2 <= n // (4 * M * N) <= 8
    s = wl.Q4Shape(M, N, K, g, 0.002, 0.02)
    d = wl.make_q4_problem(500 + N + M, s)
    t = dev(d)
    rows = sample_rows(N, 400, N) if N > 1000 else np.arange(N)
    y_ref, b = oracle.gemv_q4(d["x"], d["wq"], d["scales"], d["zeros"], g, rows=rows)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=DEV)     # contents need no initialisation
    y_ws = q4.gemv_q4(t["x"], t["wq"], t["scales"], t["zeros"], g, workspace=ws)
    y_plain = q4.gemv_q4(t["x"], t["wq"], t["scales"], t["zeros"], g, workspace=False)
    y_short = q4.gemv_q4(t["x"], t["wq"], t["scales"], t["zeros"], g, workspace=ws[:n - 16])
    torch.cuda.synchronize()
    assert_within(y_ws.cpu().numpy()[:, rows], y_ref, b, f"split M{M} N{N} K{K}")
    assert_within(y_plain.cpu().numpy()[:, rows], y_ref, b, f"unsplit M{M} N{N} K{K}")
    assert np.array_equal(y_short.cpu().numpy(), y_plain.cpu().numpy())


def test_gemv_q4_workspace_split_graph_replay():
    """The split's two launches captured in a graph: every replay, with the
    workspace overwritten between them, equals the eager result."""
    M, N, K, g = 8, 640, 14336, 128
    s = wl.Q4Shape(M, N, K, g, 0.002, 0.02)
    d = wl.make_q4_problem(77, s)
    t = dev(d)
    n = q4.gemv_q4_workspace_size(M, N, K, g)
    assert n > 0
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    y = torch.empty((M, N), device=DEV)
    eager = q4.gemv_q4(t["x"], t["wq"], t["scales"], t["zeros"], g, workspace=ws).clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q4.gemv_q4(t["x"], t["wq"], t["scales"], t["zeros"], g, out=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        q4.gemv_q4(t["x"], t["wq"], t["scales"], t["zeros"], g, out=y, workspace=ws)
    for i in range(4):
        y.fill_(float("nan"))
        ws.fill_(i * 37 % 256)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {i}"


# ---------------------------------------------------------------- every tunable geometry

GEOM_SHAPES = [(1, 14336, 4096, 128), (1, 4096, 14336, 128), (4, 515, 4096, 128),
               (8, 67, 14336, 128), (1, 896, 4864, 32), (2, 300, 8192, 128), (1, 1000, 896, 32)]


@pytest.mark.parametrize("M,N,K,g", GEOM_SHAPES, ids=[f"M{a}N{b}K{c}g{d}" for a, b, c, d in GEOM_SHAPES])
def test_every_geometry_the_tuner_may_pick(M, N, K, g):
    """Each (path, waves, K-split) that gemv_q4_set_geometry accepts gives
    results within the tolerance (sampled rows for large N)."""
    from memory_bandwidth_amd import autotune
    s = wl.Q4Shape(M, N, K, g, 0.002, 0.02)
    d = wl.make_q4_problem(400 + N, s)
    t = dev(d)
    rows = sample_rows(N, 300, N) if N > 2000 else np.arange(N)
    y_ref, b = oracle.gemv_q4(d["x"], d["wq"], d["scales"], d["zeros"], g, rows=rows)
    cands = autotune.candidates(M, N, K, g)
    assert len(cands) >= 3
    try:
        for c in cands:
            q4.gemv_q4_set_geometry(M, N, K, g, c["path"], c["waves"], c["ksplit"])
            assert q4.gemv_q4_geometry(M, N, K, g) == c["geometry"]
            y = run_q4(t, g)
            assert_within(y[:, rows], y_ref, b, f"{c['path']}/{c['waves']}/{c['ksplit']}")
    finally:
        q4.gemv_q4_clear_geometry()


# ---------------------------------------------------------------- seeded random shapes

def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.integers(1, 9))
        g = int(rng.choice([32, 128]))
        K = g * int(rng.integers(1, max(2, 12288 // g)))
        N = int(rng.integers(1, 700))
        out.append((M, N, K, g))
    return out


RANDOM_SHAPES = _random_shapes(40, 2024)


@pytest.mark.parametrize("M,N,K,g", RANDOM_SHAPES, ids=[f"M{a}N{b}K{c}g{d}" for a, b, c, d in RANDOM_SHAPES])
def test_gemv_q4_random_shapes(M, N, K, g):
    """Seeded random shapes across every planner branch (both paths, 16/32/64
    lanes per row, K-splits, x segments); each output within the tolerance."""
    s = wl.Q4Shape(M, N, K, g, 0.002, 0.02)
    d = wl.make_q4_problem(5000 + N + K, s)
    y = run_q4(dev(d), g)
    y_ref, b = oracle.gemv_q4(d["x"], d["wq"], d["scales"], d["zeros"], g)
    assert_within(y, y_ref, b, f"M{M} N{N} K{K} g{g} path {q4.gemv_q4_path(M, N, K, g)}")


# ---------------------------------------------------------------- the five workloads, every row, tuned geometry

def _oracle_all_rows(x, d, g, threads=16):
    """Every row of the oracle's GEMV, rows split over host threads."""
    import concurrent.futures
    N = d["wq"].shape[0]
    parts = [r for r in np.array_split(np.arange(N, dtype=np.int64), threads) if r.size]
    with concurrent.futures.ThreadPoolExecutor(len(parts)) as ex:
        res = list(ex.map(lambda r: oracle.gemv_q4(x, d["wq"], d["scales"], d["zeros"], g, rows=r), parts))
    return np.concatenate([a for a, _ in res], axis=1), np.concatenate([b for _, b in res], axis=1)


def _workload_cases():
    cases = [("gemv-896", wl.SMALL_896, wl.workload_seed(0), 0)]
    cases += [(f"decoder-layer {s.label}", s, wl.workload_seed(1), i) for i, s in enumerate(wl.DECODER_LAYER)]
    cases += [("lm-head", wl.LM_HEAD, wl.workload_seed(2), 0)]
    cases += [(f"ffn-8b {s.label}", s, wl.workload_seed(3), i) for M in (1, 4, 8) for i, s in enumerate(wl.ffn_8b(M))]
    cases += [("stream", wl.STREAM_SHAPE, wl.workload_seed(4), 0)]
    return cases


@pytest.fixture(scope="module")
def tuned_profile():
    """The device's tuned geometry profile applied, as the benchmark applies it."""
    from memory_bandwidth_amd import autotune
    path = autotune.default_profile_path(DEV)
    n = autotune.apply_profile(path, DEV) if os.path.exists(path) else 0
    yield n
    q4.gemv_q4_clear_geometry()
    for fmt in q4.BLOCK_FORMATS:
        q4.gemv_block_set_config(fmt, 0, 0, 0)
    q4.scan2_set_config(0, 0, 0, 0)


@pytest.mark.parametrize("case", _workload_cases(), ids=lambda c: c[0].replace(" ", "_"))
def test_workload_every_row_tuned_geometry(case, tuned_profile):
    """Each configured GEMV in the geometry the benchmark runs (the tuned
    profile applied), every output row against the oracle at the plain bound."""
    label, s, seed, index = case
    d = wl.make_q4_problem(seed, s, index=index)
    y = run_q4(dev(d), s.g)
    y_ref, b = _oracle_all_rows(d["x"], d, s.g)
    assert_within(y, y_ref, b, f"{label} (tuned profile: {tuned_profile} settings)")
