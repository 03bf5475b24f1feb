"""Pins for the CPU oracle: it is checked against the pages' definitions and
against mathematics, never against itself.

Each pin is written so that a plausible mistake in the oracle (swapped nibble
order, swapped zero-point nibble, dropped or negated zero point, wrong group
index, wrong binary16 bias, a dropped term, an operand indexed with the wrong
row) fails at least one of them; ``test_pins_catch_planted_mistakes`` plants
each of those mistakes in a copy of the oracle source and checks exactly that.
"""

import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

GOLDEN = os.path.join(ROOT, "tests", "golden", "q4_worked_examples.json")


# ---------------------------------------------------------------------------
# Test-side construction of packed matrices, written from the page's u32 view
# (eight 4-bit values per u32, value at position p in bits 4p..4p+3) rather
# than from the oracle's byte view.
# ---------------------------------------------------------------------------

def pack_codes_u32(codes: np.ndarray) -> np.ndarray:
    """codes int [N, K] (K % 8 == 0) -> wq uint8 [N, K/2] via little-endian u32 words."""
    N, K = codes.shape
    c = codes.astype(np.uint64).reshape(N, K // 8, 8)
    words = np.zeros((N, K // 8), np.uint64)
    for p in range(8):
        words |= c[:, :, p] << np.uint64(4 * p)
    return words.astype("<u4").view(np.uint8).reshape(N, K // 2)


def pack_zeros(z: np.ndarray) -> np.ndarray:
    """z int [N, G] -> uint8 [N, ceil(G/2)], even group in the low nibble."""
    N, G = z.shape
    zz = np.zeros((N, G + (G % 2)), np.int64)
    zz[:, :G] = z
    return (zz[:, 0::2] + 16 * zz[:, 1::2]).astype(np.uint8)


def dequant_flat(codes, z, s_bits, g):
    """W in float64 through the page's flat group index: group = (n*K + k) // g."""
    N, K = codes.shape
    flat = np.arange(N * K)
    grp = flat // g
    zf = z.reshape(-1)[grp]
    sf = s_bits.reshape(-1).view(np.float16).astype(np.float64)[grp]
    return ((codes.reshape(-1) - zf) * sf).reshape(N, K)


def random_case(seed, N, K, g):
    rng = np.random.default_rng(seed)
    G = K // g
    codes = rng.integers(0, 16, size=(N, K))
    z = rng.integers(0, 16, size=(N, G))
    s_bits = rng.uniform(0.002, 0.02, size=(N, G)).astype(np.float16).view(np.uint16)
    return codes, z, s_bits


# ---------------------------------------------------------------------------
# Pins.  Each takes an Oracle so the planted-mistake test can rerun them.
# ---------------------------------------------------------------------------

def pin_f16_all_patterns(o):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([o.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_golden_extract_nibble(o):
    ex = json.load(open(GOLDEN))["extract_nibble"]
    nw = -(-len(ex) // 4) * 4                           # pad to whole 32-element groups
    words = np.zeros(nw, "<u4")
    words[:len(ex)] = [int(e["packed"], 16) for e in ex]
    wq = words.view(np.uint8).reshape(1, -1)            # one row, K = 8 per word
    K = 8 * nw
    scales = np.full((1, K // 32), 0x3C00, np.uint16)   # 1.0
    zeros = np.zeros((1, (K // 32 + 1) // 2), np.uint8)
    _, codes = o.dequant(wq, scales, zeros, K, 32)
    assert codes.reshape(-1)[:8 * len(ex)].tolist() == [v for e in ex for v in e["nibbles"]]


def pin_golden_dequant(o):
    ex = json.load(open(GOLDEN))["dequant"]
    for e in ex:
        K, g = 32, 32
        codes = np.full((1, K), e["nibble"])
        wq = pack_codes_u32(codes)
        scales = np.full((1, 1), int(e["scale_f16"], 16), np.uint16)
        zeros = pack_zeros(np.full((1, 1), e["zero"]))
        w, _ = o.dequant(wq, scales, zeros, K, g)
        assert np.all(w == np.float32(e["value"])), e


def pin_golden_gemv(o):
    for e in json.load(open(GOLDEN))["gemv"]:
        K, g = e["K"], e["g"]
        codes = np.full((1, K), e["code"])
        wq = pack_codes_u32(codes)
        scales = np.full((1, K // g), int(e["scale_f16"], 16), np.uint16)
        zeros = pack_zeros(np.full((1, K // g), e["zero"]))
        x = np.ones(K, np.float32) if e["x"] == "all ones" else np.arange(1, K + 1, dtype=np.float32)
        y, _ = o.gemv_q4(x, wq, scales, zeros, g)
        assert y[0, 0] == e["y"], (e, y)


def pin_dequant_flat_index(o):
    """Random codes/zeros/scales: oracle W equals the page's flat-index dequant, bit for bit."""
    for (N, K, g, seed) in [(3, 64, 32, 1), (5, 384, 128, 2), (2, 96, 32, 3)]:
        codes, z, s_bits = random_case(seed, N, K, g)
        w, c = o.dequant(pack_codes_u32(codes), s_bits, pack_zeros(z), K, g)
        assert np.array_equal(c, codes.astype(np.uint8))
        ref = dequant_flat(codes, z, s_bits, g).astype(np.float32)
        assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))


def pin_one_hot_x(o):
    """x = e_k makes y[n] = W(n, k) exactly: pins orientation and group index."""
    N, K, g = 4, 512, 128
    codes, z, s_bits = random_case(7, N, K, g)
    wq, zeros = pack_codes_u32(codes), pack_zeros(z)
    Wref = dequant_flat(codes, z, s_bits, g)
    for k in [0, 1, 7, 8, 127, 128, 129, 255, 256, 383, 384, 511]:
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        y, b = o.gemv_q4(x, wq, s_bits, zeros, g)
        assert np.array_equal(y[0], Wref[:, k]), k
        assert np.array_equal(b[0], np.abs(Wref[:, k])), k


def pin_zero_point_groups(o):
    """Distinct zero point per group (groups 0..3), one-hot x inside each group."""
    N, K, g = 2, 128, 32
    codes = np.full((N, K), 15)
    z = np.array([[1, 4, 9, 13], [0, 15, 2, 7]])
    s_bits = np.full((N, 4), 0x3C00, np.uint16)
    wq, zeros = pack_codes_u32(codes), pack_zeros(z)
    for j in range(4):
        x = np.zeros((1, K), np.float32)
        x[0, j * g + 5] = 1.0
        y, _ = o.gemv_q4(x, wq, s_bits, zeros, g)
        assert y[0].tolist() == [15 - z[0, j], 15 - z[1, j]], j


def pin_closed_form_z8(o):
    """z = 8, q = c, x = 1: y[n] = (c - 8) * g * sum_j s(n, j), exact in f64."""
    N, K, g = 6, 1024, 128
    rng = np.random.default_rng(11)
    s_bits = rng.uniform(0.002, 0.01, size=(N, K // g)).astype(np.float16).view(np.uint16)
    s = s_bits.view(np.float16).astype(np.float64)
    zeros = np.full((N, (K // g + 1) // 2), 0x88, np.uint8)
    x = np.ones((1, K), np.float32)
    for c in [0, 3, 8, 15]:
        wq = np.full((N, K // 2), c * 0x11, np.uint8)
        y, _ = o.gemv_q4(x, wq, s_bits, zeros, g)
        assert np.array_equal(y[0], (c - 8) * g * s.sum(axis=1)), c
        w, _ = o.dequant(wq, s_bits, zeros, K, g)
        assert np.array_equal(w, np.repeat(((c - 8) * s).astype(np.float32), g, axis=1))


def pin_q_equals_z(o):
    """q = z everywhere: W is +0 and y is exactly 0 for any x."""
    N, K, g = 5, 256, 32
    z = np.random.default_rng(5).integers(0, 16, size=(N, K // g))
    codes = np.repeat(z, g, axis=1)
    s_bits = np.full((N, K // g), 0x2E66, np.uint16)
    x = workloads.make_x(3, 3, K)
    y, b = o.gemv_q4(x, pack_codes_u32(codes), s_bits, pack_zeros(z), g)
    assert np.all(y == 0.0) and np.all(b == 0.0)
    w, _ = o.dequant(pack_codes_u32(codes), s_bits, pack_zeros(z), K, g)
    assert np.all(w.view(np.uint32) == 0)


def pin_round_trip(o):
    """w = (q - z) s exactly; quantize(w) recovers q and dequant(quantize(w)) == w."""
    N, K, g = 7, 256, 128
    codes, z, s_bits = random_case(13, N, K, g)
    wq, zeros = pack_codes_u32(codes), pack_zeros(z)
    w, _ = o.dequant(wq, s_bits, zeros, K, g)
    wq2 = o.quantize(w, s_bits, zeros, g)
    assert np.array_equal(wq2, wq)
    w2, _ = o.dequant(wq2, s_bits, zeros, K, g)
    assert np.array_equal(w2.view(np.uint32), w.view(np.uint32))


def pin_gemv_vs_numpy(o):
    """Random problem: y agrees with numpy float64 matmul of the flat-index dequant."""
    for (M, N, K, g, seed) in [(3, 37, 256, 32, 21), (8, 19, 512, 128, 22)]:
        codes, z, s_bits = random_case(seed, N, K, g)
        x = workloads.make_x(seed, M, K)
        y, b = o.gemv_q4(x, pack_codes_u32(codes), s_bits, pack_zeros(z), g)
        W = dequant_flat(codes, z, s_bits, g)
        ref = x.astype(np.float64) @ W.T
        bref = np.abs(x.astype(np.float64)) @ np.abs(W).T
        assert np.all(np.abs(y - ref) <= 1e-12 * bref + 1e-300)
        assert np.allclose(b, bref, rtol=1e-12, atol=0)


def pin_integer_exact(o):
    """Power-of-two scales and integer x: y * 2^10 is an integer the test computes exactly."""
    M, N, K, g = 3, 11, 640, 32
    d = workloads.make_exact_problem(31, M, N, K, g)
    y, _ = o.gemv_q4(d["x"], d["wq"], d["scales"], d["zeros"], g)
    # decode the packed arrays through the u32 view, independently of the oracle
    words = d["wq"].reshape(N, K // 8, 4).copy().view("<u4").reshape(N, K // 8).astype(np.int64)
    codes = np.stack([(words >> (4 * p)) & 15 for p in range(8)], axis=-1).reshape(N, K)
    zb = d["zeros"].astype(np.int64)
    z = np.stack([zb & 15, zb >> 4], axis=-1).reshape(N, -1)[:, :K // g]
    e = -np.log2(d["scales"].view(np.float16).astype(np.float64)).astype(np.int64)
    num = (codes - np.repeat(z, g, axis=1)) * np.repeat(1 << (10 - e), g, axis=1)
    exact = d["x"].astype(np.int64) @ num.T                 # = y * 2^10
    assert np.array_equal(y * 1024.0, exact.astype(np.float64))


def pin_gemv_f32(o):
    rng = np.random.default_rng(41)
    x = rng.standard_normal((4, 300)).astype(np.float32)
    w = rng.standard_normal((23, 300)).astype(np.float32)
    y, b = o.gemv_f32(x, w)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    bref = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    assert np.all(np.abs(y - ref) <= 1e-12 * bref)
    assert np.allclose(b, bref, rtol=1e-12, atol=0)
    xi = rng.integers(-3, 4, size=(2, 64)).astype(np.float32)
    wi = rng.integers(-100, 101, size=(9, 64)).astype(np.float32)
    yi, _ = o.gemv_f32(xi, wi)
    assert np.array_equal(yi, (xi.astype(np.int64) @ wi.astype(np.int64).T).astype(np.float64))
    rows = np.array([8, 0, 3])
    yr, _ = o.gemv_f32(x, w, rows)
    assert np.array_equal(yr, y[:, rows])


def pin_rows_subset(o):
    N, K, g = 9, 256, 32
    codes, z, s_bits = random_case(51, N, K, g)
    x = workloads.make_x(51, 2, K)
    args = (x, pack_codes_u32(codes), s_bits, pack_zeros(z), g)
    y, b = o.gemv_q4(*args)
    rows = np.array([8, 2, 2, 0])
    yr, br = o.gemv_q4(*args, rows=rows)
    assert np.array_equal(yr, y[:, rows]) and np.array_equal(br, b[:, rows])


def pin_buffer_sum(o):
    s, a = o.buffer_sum(np.ones(1 << 20, np.float32))
    assert s == float(1 << 20) and a == float(1 << 20)
    buf = workloads.make_probe_buffer(100003) - 0.5
    s, a = o.buffer_sum(buf)
    assert abs(s - buf.astype(np.float64).sum()) <= 1e-12 * a
    assert abs(a - np.abs(buf.astype(np.float64)).sum()) <= 1e-12 * a


PINS = [pin_f16_all_patterns, pin_golden_extract_nibble, pin_golden_dequant,
        pin_golden_gemv, pin_dequant_flat_index, pin_one_hot_x, pin_zero_point_groups,
        pin_closed_form_z8, pin_q_equals_z, pin_round_trip, pin_gemv_vs_numpy,
        pin_integer_exact, pin_gemv_f32, pin_rows_subset, pin_buffer_sum]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(oracle.load())


# ---------------------------------------------------------------------------
# Planted mistakes: each mutation of the oracle source must fail some pin.
# ---------------------------------------------------------------------------

MUTATIONS = {
    "code_nibble_swapped": ("static int code_at", "(k & 1) ? (b >> 4) : (b & 0x0F)",
                            "(k & 1) ? (b & 0x0F) : (b >> 4)"),
    "zero_nibble_swapped": ("static int zero_at", "(j & 1) ? (b >> 4) : (b & 0x0F)",
                            "(j & 1) ? (b & 0x0F) : (b >> 4)"),
    "zero_dropped": ("static double weight_at", "(double)(q - z) * s", "(double)(q) * s"),
    "zero_sign_flipped": ("static double weight_at", "(double)(q - z) * s", "(double)(z - q) * s"),
    "group_index_fixed_32": ("static double weight_at", "int64_t j = k / g;", "int64_t j = k / 32;"),
    "zero_row_stride_G": ("static int zero_at", "int64_t zb = (G + 1) / 2;", "int64_t zb = G;"),
    "f16_bias_off_by_one": ("double q4ref_f16_to_f64", "e - 25", "e - 24"),
    "f16_subnormal_scale": ("double q4ref_f16_to_f64", "ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "gemv_last_term_dropped": ("void q4ref_gemv_q4_rows", "for (int64_t k = 0; k < K; ++k)",
                               "for (int64_t k = 0; k < K - 1; ++k)"),
    "gemv_x_row_ignored": ("void q4ref_gemv_q4_rows", "(double)x[m * K + k]", "(double)x[k]"),
    "gemv_weight_transposed": ("void q4ref_gemv_q4_rows", "weight_at(wq, scales, zeros, K, g, n, k)",
                               "weight_at(wq, scales, zeros, K, g, k % N, n % K)"),
    "f32_operand_row": ("void q4ref_gemv_f32_rows", "(double)w[n * K + k]", "(double)w[k]"),
    "sum_abs_missing": ("void q4ref_sum", "a += fabs((double)buf[i]);", "a += (double)buf[i];"),
}


def _mutant(tmp_path, name):
    anchor, old, new = MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "q4ref.c")).read()
    i = src.index(anchor)
    j = src.index(old, i)
    mutated = src[:j] + new + src[j + len(old):]
    path = tmp_path / f"{name}.c"
    path.write_text(mutated)
    return oracle.Oracle(oracle.build(src=str(path), out=str(tmp_path / f"lib{name}.so")))


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistakes(tmp_path, name):
    o = _mutant(tmp_path, name)
    caught = []
    for pin in PINS:
        try:
            pin(o)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"


def test_oracle_under_sanitizers(tmp_path):
    """Build the oracle with ASan/UBSan into a small C driver and run it on
    exact-size heap buffers, so any out-of-bounds access aborts."""
    driver = tmp_path / "drive.c"
    driver.write_text(r'''
#include <stdint.h>
#include <stdlib.h>
#include <stdio.h>
void q4ref_dequant(const uint8_t*, const uint16_t*, const uint8_t*, int64_t, int64_t, int64_t, float*, uint8_t*);
void q4ref_gemv_q4(const float*, const uint8_t*, const uint16_t*, const uint8_t*, int64_t, int64_t, int64_t, int64_t, double*, double*);
void q4ref_gemv_f32(const float*, const float*, int64_t, int64_t, int64_t, double*, double*);
void q4ref_quantize(const float*, const uint16_t*, const uint8_t*, int64_t, int64_t, int64_t, uint8_t*);
void q4ref_sum(const float*, int64_t, double*, double*);
int main(void) {
  const int64_t shapes[][4] = {{1, 3, 96, 32}, {3, 5, 384, 128}, {2, 7, 160, 32}};
  for (int t = 0; t < 3; ++t) {
    int64_t M = shapes[t][0], N = shapes[t][1], K = shapes[t][2], g = shapes[t][3];
    int64_t G = K / g, ZB = (G + 1) / 2;
    uint8_t *wq = malloc(N * K / 2), *zeros = malloc(N * ZB), *codes = malloc(N * K), *wq2 = calloc(N * K / 2, 1);
    uint16_t *sc = malloc(N * G * 2);
    float *x = malloc(M * K * 4), *w = malloc(N * K * 4);
    double *y = malloc(M * N * 8), *b = malloc(M * N * 8), s, a;
    for (int64_t i = 0; i < N * K / 2; ++i) wq[i] = (uint8_t)(i * 37 + 11);
    for (int64_t i = 0; i < N * ZB; ++i) zeros[i] = (uint8_t)(i * 53 + 7);
    for (int64_t i = 0; i < N * G; ++i) sc[i] = (uint16_t)(0x2000 + i);
    for (int64_t i = 0; i < M * K; ++i) x[i] = (float)(i % 7) - 3.0f;
    q4ref_dequant(wq, sc, zeros, N, K, g, w, codes);
    q4ref_gemv_q4(x, wq, sc, zeros, M, N, K, g, y, b);
    q4ref_gemv_f32(x, w, M, N, K, y, b);
    q4ref_quantize(w, sc, zeros, N, K, g, wq2);
    q4ref_sum(w, N * K, &s, &a);
    for (int64_t i = 0; i < N * K / 2; ++i) if (wq2[i] != wq[i]) { printf("round trip\n"); return 1; }
    free(wq); free(zeros); free(codes); free(wq2); free(sc); free(x); free(w); free(y); free(b);
  }
  printf("ok\n");
  return 0;
}
''')
    exe = tmp_path / "drive"
    subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-std=c99", "-o", str(exe), str(driver),
                    os.path.join(ROOT, "oracle", "q4ref.c"), "-lm"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr


# ---------------------------------------------------------------- SwiGLU combine

def test_silu_odd_part_is_the_identity():
    """silu(v) - silu(-v) = v (v sigma(v) + v sigma(-v) = v): fixes the sign
    of the exponent and the 1 + e^-v denominator."""
    v = np.concatenate([np.linspace(-30, 30, 601), [1e-8, -1e-8, 100.0, -250.0, 700.0]])
    d = oracle.silu(v) - oracle.silu(-v)
    assert np.allclose(d, v, rtol=1e-14, atol=0)


def test_silu_special_values():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1e-9) == pytest.approx(0.5e-9, rel=1e-8)      # slope 1/2 at 0
    assert oracle.silu(50.0) == pytest.approx(50.0, rel=1e-20)
    assert 0 > oracle.silu(-50.0) > -50.0 * 2e-22                      # -50 e^-50
    assert oracle.silu(-800.0) == 0.0                                  # e^800 overflows: -0


def test_silu_slope_bound_used_by_the_tolerance():
    """The SwiGLU tolerance takes |silu'| <= 1.1; the true maximum is about 1.0998."""
    v = np.linspace(-20, 20, 400001)
    slope = np.diff(oracle.silu(v)) / np.diff(v)
    assert 1.09 < slope.max() < 1.1 and slope.min() > -0.11


def test_swiglu_invariants():
    """gate == up gives silu(g) g >= 0; an up matrix with q == z gives exactly 0;
    a gate with q == z gives exactly 0."""
    s = workloads.Q4Shape(2, 37, 256, 32, 0.005, 0.02)
    d = workloads.make_q4_problem(21, s)
    mat = (d["wq"], d["scales"], d["zeros"])
    y, tol = oracle.swiglu(d["x"], mat, mat, s.g)
    assert (y >= 0).all() and (tol > 0).all()
    z = np.stack([d["zeros"] & 15, d["zeros"] >> 4], -1).reshape(s.N, -1)[:, :s.K // s.g]
    codes = np.repeat(z, s.g, axis=1).astype(np.uint8)
    flat = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    dead = (flat, d["scales"], d["zeros"])
    assert np.all(oracle.swiglu(d["x"], mat, dead, s.g)[0] == 0)
    assert np.all(oracle.swiglu(d["x"], dead, mat, s.g)[0] == 0)


def test_fused_rows_are_the_separate_gemvs():
    """Matrices stored one after another (workloads.fuse_rows) give, row for
    row, the GEMVs of the separate matrices: the layout mixes nothing."""
    mats = [workloads.make_q4_weights(22, n, 256, 32, 0.005, 0.02, index=i)
            for i, n in enumerate((40, 8, 8))]
    x = workloads.make_x(22, 2, 256)
    fused = workloads.fuse_rows(*mats)
    y, b = oracle.gemv_q4(x, fused["wq"], fused["scales"], fused["zeros"], 32)
    parts = [oracle.gemv_q4(x, m["wq"], m["scales"], m["zeros"], 32) for m in mats]
    assert np.array_equal(y, np.concatenate([p[0] for p in parts], axis=1))
    assert np.array_equal(b, np.concatenate([p[1] for p in parts], axis=1))
