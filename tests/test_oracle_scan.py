"""Pins for the 2-bit scan oracle (oracle/scan.py, oracle/scanref.c).

The scan computes score[v, q] = sum_d lut[q, d, code(v, d)] over 2-bit codes
packed 16 per little-endian u32.  The pins check it against closed forms
(constant codes reduce it to one table column's sum; a one-hot table counts
matching codes), hand-packed words with a hand-summed score, and exact
integer arithmetic for a table of the form query * level.  Codes are packed
here from integer arrays by array operations, independently of the oracle's
per-element extraction.  ``test_scan_pins_catch_planted_mistakes`` plants
plausible mistakes in a copy of the oracle and checks each is caught.
"""

import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from oracle import scan  # noqa: E402
import workloads as wl  # noqa: E402


def pack_codes(c: np.ndarray) -> np.ndarray:
    """int codes [V, D] in 0..3 -> uint32 [V, D/16], dimension 16w + i in bits 2i, 2i+1."""
    V, D = c.shape
    c = c.astype(np.uint64).reshape(V, D // 16, 16)
    words = (c << (2 * np.arange(16, dtype=np.uint64))).sum(axis=2)
    return words.astype(np.uint32)


def pin_constant_codes(o):
    rng = np.random.default_rng(1)
    lut = rng.standard_normal((3, 48, 4)).astype(np.float32)
    for c0 in range(4):
        codes = np.full((5, 3), 0x55555555 * c0, np.uint32)
        s, b = o.scan(codes, lut)
        want = lut[:, :, c0].astype(np.float64).sum(axis=1)
        assert np.allclose(s, np.broadcast_to(want, s.shape), rtol=1e-12, atol=1e-12)
        assert np.allclose(b, np.abs(lut[:, :, c0].astype(np.float64)).sum(axis=1), rtol=1e-12)


def pin_one_hot_table(o):
    rng = np.random.default_rng(2)
    c = rng.integers(0, 4, (40, 64))
    codes = pack_codes(c)
    for d0, c0, q0 in ((0, 3, 1), (17, 1, 0), (63, 2, 2), (31, 0, 1)):
        lut = np.zeros((3, 64, 4), np.float32)
        lut[q0, d0, c0] = 1.0
        s, _ = o.scan(codes, lut)
        want = np.zeros((40, 3))
        want[:, q0] = (c[:, d0] == c0)
        assert np.array_equal(s, want), (d0, c0, q0)


def pin_hand_words(o):
    """D = 16, one word 0xE40000E4: dimensions 0..3 and 12..15 hold codes
    0, 1, 2, 3, dimensions 4..11 code 0.  With lut[q, d, c] = c + 4d (q = 0)
    the score is (0 + 5 + 10 + 15) + 4 * (4 + ... + 11) + (48 + 53 + 58 + 63)
    = 30 + 240 + 222 = 492; with lut = 1 everywhere (q = 1) it is 16."""
    lut = np.zeros((2, 16, 4), np.float32)
    lut[0] = np.arange(4)[None, :] + 4 * np.arange(16)[:, None]
    lut[1] = 1.0
    s, _ = o.scan(np.array([[0xE40000E4]], np.uint32), lut)
    assert np.array_equal(s, [[492.0, 16.0]])


def pin_query_level_dot(o):
    """lut[q, d, c] = query[q, d] * level[d, c] with small integers: the score
    is the dot product of query q with the dequantised vector, exactly."""
    rng = np.random.default_rng(3)
    V, D, Q = 23, 96, 8
    c = rng.integers(0, 4, (V, D))
    query = rng.integers(-3, 4, (Q, D))
    level = rng.integers(-2, 3, (D, 4))
    lut = (query[:, :, None] * level[None, :, :]).astype(np.float32)
    s, _ = o.scan(pack_codes(c), lut)
    want = [[sum(int(query[q, d]) * int(level[d, c[v, d]]) for d in range(D)) for q in range(Q)]
            for v in range(V)]
    assert np.array_equal(s, np.array(want, np.float64))


def pin_rows_subset(o):
    codes = wl.make_scan_codes(4, 30, 64)
    lut = wl.make_scan_lut(4, 3, 64)
    s, b = o.scan(codes, lut)
    rows = np.array([29, 0, 7])
    s2, b2 = o.scan(codes, lut, rows)
    assert np.array_equal(s2, s[rows]) and np.array_equal(b2, b[rows])
    assert np.all(b >= np.abs(s))


PINS = [pin_constant_codes, pin_one_hot_table, pin_hand_words, pin_query_level_dot, pin_rows_subset]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_scan_oracle_pin(pin):
    pin(scan.load())


def test_generators():
    codes = wl.make_scan_codes(5, 100, 768)
    lut = wl.make_scan_lut(5, 8, 768)
    assert codes.shape == (100, 48) and codes.dtype == np.uint32
    assert lut.shape == (8, 768, 4) and lut.dtype == np.float32 and np.all(np.isfinite(lut))
    # every code value occurs at every dimension
    c = (codes[:, :, None] >> (2 * np.arange(16, dtype=np.uint32))) & 3
    assert set(np.unique(c)) == {0, 1, 2, 3}


MUTATIONS = {
    "bit_order_reversed": ("static int code_at", "(w >> (2 * (d % 16)))", "(w >> (2 * (15 - d % 16)))"),
    "word_index": ("static int code_at", "codes[v * (D / 16) + d / 16]", "codes[v * (D / 16) + d / 32]"),
    "one_bit": ("static int code_at", "& 3u", "& 1u"),
    "lut_transposed": ("void scanref_rows", "lut[(q * D + d) * 4", "lut[(d * Q + q) * 4"),
    "bound_abs_dropped": ("void scanref_rows", "b += fabs(t);", "b += t;"),
    "last_term_dropped": ("void scanref_rows", "for (int64_t d = 0; d < D; ++d)",
                          "for (int64_t d = 0; d + 1 < D; ++d)"),
    "vector_stride": ("static int code_at", "codes[v * (D / 16)", "codes[v * (D / 32)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_scan_pins_catch_planted_mistakes(tmp_path, name):
    anchor, old, new = MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "scanref.c")).read()
    i = src.index(anchor)
    j = src.index(old, i)
    path = tmp_path / f"{name}.c"
    path.write_text(src[:j] + new + src[j + len(old):])
    o = scan.ScanOracle(oracle.build(src=str(path), out=str(tmp_path / f"lib{name}.so")))
    caught = []
    for pin in PINS:
        try:
            pin(o)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
