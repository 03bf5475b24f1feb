"""Pins for the block-format oracle (oracle/blocks.py, oracle/blockref.c).

The page fixes only each format's geometry; the decoding is the published
definition of the GGML formats of those names.  The pins check the oracle
against the page's geometry table, against blocks packed here from integer
fields (the packers are the inverse of the format rules, written as array
operations rather than per-element decoding), against hand-worked blocks, and
against reductions to other, separately pinned results: Q4_0 is the int4
format with g = 32 and zero point 8, Q5_K without its fifth bits is Q4_K, and
Q8_0 with d = 1 is an integer dot product.
``test_block_pins_catch_planted_mistakes`` plants plausible mistakes in a copy
of the oracle source and checks that some pin fails for each.
"""

import json
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from oracle import blocks  # noqa: E402
import workloads as wl  # noqa: E402

GOLDEN = os.path.join(ROOT, "tests", "golden", "block_geometry.json")
CODES = {"q4_0": blocks.Q4_0, "q8_0": blocks.Q8_0, "q4_k": blocks.Q4_K,
         "q5_k": blocks.Q5_K, "q6_k": blocks.Q6_K}


def f16_bits(v) -> int:
    return int(np.float16(v).view(np.uint16))


def f16_val(bits) -> float:
    return float(np.uint16(bits).view(np.float16))


def le16(bits) -> np.ndarray:
    return np.array([bits & 0xFF, bits >> 8], np.uint8)


# ---------------------------------------------------------------------------
# Packers: integer fields -> block bytes.
# ---------------------------------------------------------------------------

def pack_q4_0(d, q):
    """q: 32 codes 0..15; element i < 16 low nibble of byte i, 16 + i high."""
    q = np.asarray(q, np.uint8)
    return np.concatenate([le16(d), q[:16] | (q[16:] << 4)])


def pack_q8_0(d, q):
    return np.concatenate([le16(d), np.asarray(q, np.int8).view(np.uint8)])


def pack_scale_min(s, m):
    """Eight 6-bit scales and mins -> 12 bytes: bytes 0-3 and 4-7 keep the
    low six bits of s[0..3] and m[0..3] with the top two bits of s[4..7] and
    m[4..7] above them; bytes 8-11 keep the low nibbles of s[4..7] and
    m[4..7]."""
    s, m = np.asarray(s, np.uint8), np.asarray(m, np.uint8)
    return np.concatenate([s[:4] | ((s[4:] >> 4) << 6),
                           m[:4] | ((m[4:] >> 4) << 6),
                           (s[4:] & 15) | ((m[4:] & 15) << 4)]).astype(np.uint8)


def _k_nibbles(q4):
    """256 four-bit values -> 128 bytes: element 64p + l low, 64p + 32 + l high."""
    q = np.asarray(q4, np.uint8).reshape(4, 2, 32)
    return (q[:, 0, :] | (q[:, 1, :] << 4)).reshape(128)


def pack_q4_k(d, dmin, s, m, q):
    return np.concatenate([le16(d), le16(dmin), pack_scale_min(s, m), _k_nibbles(q)])


def pack_q5_k(d, dmin, s, m, q):
    """q: 256 values 0..31; bit 4 of element 32j + l is bit j of qh[l]."""
    q = np.asarray(q, np.int64)
    high = (q >> 4).reshape(8, 32)
    qh = (high << np.arange(8)[:, None]).sum(axis=0).astype(np.uint8)
    return np.concatenate([le16(d), le16(dmin), pack_scale_min(s, m), qh, _k_nibbles(q & 15)])


def pack_q6_k(d, sc, q):
    """q: 256 values 0..63, sc: 16 int8.  Element 128h + 32t + l keeps its low
    nibble in nibble t // 2 of ql[64h + 32(t % 2) + l] and its top two bits
    in bits 2t, 2t + 1 of qh[32h + l]."""
    q = np.asarray(q, np.int64).reshape(2, 4, 32)       # [h, t, l]
    low, top = q & 15, q >> 4
    ql = np.zeros((2, 2, 32), np.int64)                 # [h, t % 2, l]
    for t in range(4):
        ql[:, t % 2, :] |= low[:, t, :] << (4 * (t // 2))
    qh = sum(top[:, t, :] << (2 * t) for t in range(4))  # [h, l]
    return np.concatenate([ql.reshape(128).astype(np.uint8), qh.reshape(64).astype(np.uint8),
                           np.asarray(sc, np.int8).view(np.uint8), le16(d)])


def random_block(fmt, rng):
    """(block bytes, exact weights float64 [elems], tolerance magnitudes [elems])."""
    d = f16_bits(rng.uniform(0.01, 0.05) * rng.choice([-1, 1]))
    dv = f16_val(d)
    if fmt == "q4_0":
        q = rng.integers(0, 16, 32)
        w = dv * (q - 8.0)
        return pack_q4_0(d, q), w, np.abs(w)
    if fmt == "q8_0":
        q = rng.integers(-128, 128, 32)
        w = dv * q
        return pack_q8_0(d, q), w, np.abs(w)
    if fmt in ("q4_k", "q5_k"):
        dmin = f16_bits(rng.uniform(0.01, 0.05))
        s, m = rng.integers(0, 64, 8), rng.integers(0, 64, 8)
        q = rng.integers(0, 16 if fmt == "q4_k" else 32, 256)
        j = np.arange(256) // 32
        t1 = dv * s[j] * q
        t2 = f16_val(dmin) * m[j]
        pack = pack_q4_k if fmt == "q4_k" else pack_q5_k
        return pack(d, dmin, s, m, q), t1 - t2, np.abs(t1) + np.abs(t2)
    if fmt == "q6_k":
        sc = rng.integers(-128, 128, 16)
        q = rng.integers(0, 64, 256)
        w = dv * sc[np.arange(256) // 16] * (q - 32.0)
        return pack_q6_k(d, sc, q), w, np.abs(w)
    raise ValueError(fmt)


def random_matrix(fmt, N, nblk, seed):
    rng = np.random.default_rng(seed)
    rows, ws, mags = [], [], []
    for _ in range(N):
        parts = [random_block(fmt, rng) for _ in range(nblk)]
        rows.append(np.concatenate([p[0] for p in parts]))
        ws.append(np.concatenate([p[1] for p in parts]))
        mags.append(np.concatenate([p[2] for p in parts]))
    return np.stack(rows), np.stack(ws), np.stack(mags)


def exact_weights(o, fmt, w, K):
    """W[n, k] in f64 from the oracle's GEMV against the identity: row k of x
    picks out column k exactly."""
    y, _ = o.gemv(CODES[fmt], np.eye(K, dtype=np.float32), w)
    return y.T


# ---------------------------------------------------------------------------
# Pins.  Each takes a BlockOracle so the planted-mistake test can rerun them.
# ---------------------------------------------------------------------------

def pin_geometry(o):
    g = json.load(open(GOLDEN))["formats"]
    for name, code in CODES.items():
        assert o.geometry(code) == tuple(g[name]), name
        assert wl.BLOCK_FORMATS[name][1:3] == tuple(g[name]), name
    with pytest.raises(ValueError):
        o.geometry(9)


def pin_packed_fields(o):
    for i, fmt in enumerate(CODES):
        e = o.geometry(CODES[fmt])[0]
        nblk = 2 if e == 256 else 6
        w, W, _ = random_matrix(fmt, 3, nblk, 100 + i)
        K = nblk * e
        got = exact_weights(o, fmt, w, K)
        assert np.array_equal(got, W), fmt
        assert np.array_equal(o.dequant(CODES[fmt], w, K), W.astype(np.float32)), fmt


def pin_bound(o):
    for i, fmt in enumerate(CODES):
        e = o.geometry(CODES[fmt])[0]
        nblk = 2 if e == 256 else 4
        w, W, A = random_matrix(fmt, 4, nblk, 200 + i)
        K = nblk * e
        x = np.random.default_rng(7).standard_normal((2, K)).astype(np.float32)
        y, b = o.gemv(CODES[fmt], x, w)
        xd = x.astype(np.float64)
        assert np.allclose(y, xd @ W.T, rtol=1e-12, atol=1e-12), fmt
        assert np.allclose(b, np.abs(xd) @ A.T, rtol=1e-12, atol=1e-12), fmt
        rows = np.array([3, 0])
        y2, b2 = o.gemv(CODES[fmt], x, w, rows)
        assert np.array_equal(y2, y[:, rows]) and np.array_equal(b2, b[:, rows]), fmt


def pin_q4_k_hand_block(o):
    """d = 1, dmin = 0.5, every qs byte 0x31 (low code 1, high code 3).
    Scale bytes and the (scale, min) each sub-block j reads from them:
      j 0-3: low six bits of bytes 0-3 (0xC1 0x02 0x43 0x84) and 4-7
             (0x05 0x46 0x87 0xC8): (1, 5) (2, 6) (3, 7) (4, 8)
      j 4-7: low nibble of bytes 8-11 (0x9A 0xBC 0xDE 0xF1) under the top two
             bits of bytes 0-3, high nibble under those of bytes 4-7:
             (10 + 3*16, 9 + 0*16) = (58, 9), (12 + 0, 11 + 16) = (12, 27),
             (14 + 16, 13 + 32) = (30, 45), (1 + 32, 15 + 48) = (33, 63)
    w = s * q - 0.5 * m, q = 1 in even and 3 in odd sub-blocks:
      -1.5, 3, -0.5, 8, 53.5, 22.5, 7.5, 67.5."""
    sc = [0xC1, 0x02, 0x43, 0x84, 0x05, 0x46, 0x87, 0xC8, 0x9A, 0xBC, 0xDE, 0xF1]
    blk = np.concatenate([le16(0x3C00), le16(0x3800), np.array(sc, np.uint8),
                          np.full(128, 0x31, np.uint8)])
    want = np.repeat([-1.5, 3, -0.5, 8, 53.5, 22.5, 7.5, 67.5], 32)
    assert np.array_equal(exact_weights(o, "q4_k", blk[None], 256)[0], want)
    # The same header with qh all ones: each element gains 16 * s_j (d = 1).
    blk5 = np.concatenate([blk[:16], np.full(32, 0xFF, np.uint8), blk[16:]])
    s = np.repeat([1, 2, 3, 4, 58, 12, 30, 33], 32)
    assert np.array_equal(exact_weights(o, "q5_k", blk5[None], 256)[0], want + 16 * s)


def pin_q6_k_hand_block(o):
    """d = 0.5, scales sc[i] = i - 8, every ql/qh byte zero except element
    229 = 128 * 1 + 32 * 3 + 5: its low nibble is the high nibble of ql[101]
    (0xD0 -> 13) and its top bits are bits 6-7 of qh[37] (0x80 -> 2), so
    q = 13 + 32 = 45 and w = 0.5 * sc[14] * (45 - 32) = 0.5 * 6 * 13 = 39.
    Every other element has q = 0: w = 0.5 * sc[e // 16] * -32."""
    ql = np.zeros(128, np.uint8)
    qh = np.zeros(64, np.uint8)
    ql[101], qh[37] = 0xD0, 0x80
    sc = (np.arange(16) - 8).astype(np.int8).view(np.uint8)
    blk = np.concatenate([ql, qh, sc, le16(0x3800)])
    want = 0.5 * (np.arange(256) // 16 - 8) * -32.0
    want[229] = 39.0
    assert np.array_equal(exact_weights(o, "q6_k", blk[None], 256)[0], want)


def pin_q4_0_is_int4_g32_zero8(o):
    """Q4_0 is the int4 format with g = 32, zero point 8 and scale d, with
    its codes in another order: the two oracles give identical GEMVs."""
    N, K = 5, 256
    d = wl.make_q4_weights(11, N, K, 32, 0.005, 0.02)
    d["zeros"][:] = 0x88
    codes = np.empty((N, K), np.int64)
    codes[:, 0::2] = d["wq"] & 15
    codes[:, 1::2] = d["wq"] >> 4
    rows = []
    for n in range(N):
        rows.append(np.concatenate([pack_q4_0(int(d["scales"][n, b]), codes[n, 32 * b:32 * b + 32])
                                    for b in range(K // 32)]))
    w = np.stack(rows)
    x = wl.make_x(12, 2, K)
    y_blk, _ = o.gemv(blocks.Q4_0, x, w)
    y_q4, _ = oracle.gemv_q4(x, d["wq"], d["scales"], d["zeros"], 32)
    assert np.array_equal(y_blk, y_q4)


def pin_q8_0_integer_exact(o):
    """d = 1: y is the integer dot product of the int8 codes with integer x."""
    rng = np.random.default_rng(13)
    K = 320
    q = rng.integers(-128, 128, (3, K))
    w = np.stack([np.concatenate([pack_q8_0(0x3C00, q[n, 32 * b:32 * b + 32])
                                  for b in range(K // 32)]) for n in range(3)])
    x = rng.integers(-3, 4, (2, K))
    y, _ = o.gemv(blocks.Q8_0, x.astype(np.float32), w)
    want = [[sum(int(a) * int(b) for a, b in zip(x[m], q[n])) for n in range(3)] for m in range(2)]
    assert np.array_equal(y, np.array(want, np.float64))


def pin_q5_k_without_fifth_bits_is_q4_k(o):
    rng = np.random.default_rng(14)
    s, m = rng.integers(0, 64, 8), rng.integers(0, 64, 8)
    q = rng.integers(0, 16, 256)
    b4 = pack_q4_k(0x2E66, 0x2A00, s, m, q)
    b5 = pack_q5_k(0x2E66, 0x2A00, s, m, q)
    assert np.array_equal(b5[48:], b4[16:]) and not b5[16:48].any()
    assert np.array_equal(exact_weights(o, "q5_k", b5[None], 256),
                          exact_weights(o, "q4_k", b4[None], 256))


PINS = [pin_geometry, pin_packed_fields, pin_bound, pin_q4_k_hand_block, pin_q6_k_hand_block,
        pin_q4_0_is_int4_g32_zero8, pin_q8_0_integer_exact, pin_q5_k_without_fifth_bits_is_q4_k]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_block_oracle_pin(pin):
    pin(blocks.load())


def test_generator_fields_are_finite():
    """The seeded generator writes finite, positive binary16 values into every
    field that scales a block, so no decoded weight is infinite or NaN."""
    for name, (code, e, b, offs) in wl.BLOCK_FORMATS.items():
        w = wl.make_block_weights(3, name, 4, 512)
        assert w.shape == (4, 512 // e * b)
        blk = w.reshape(4, 512 // e, b)
        for off in offs:
            v = blk[:, :, off:off + 2].copy().view(np.float16).astype(np.float64)
            assert np.all(np.isfinite(v)) and np.all(v > 0), name
        assert np.all(np.isfinite(blocks.dequant(code, w, 512))), name


# ---------------------------------------------------------------------------
# Planted mistakes: each mutation of the oracle source must fail some pin.
# ---------------------------------------------------------------------------

MUTATIONS = {
    "q4_0_halves_swapped": ("case BF_Q4_0", "(e < 16) ? (b[2 + i] & 15) : (b[2 + i] >> 4)",
                            "(e < 16) ? (b[2 + i] >> 4) : (b[2 + i] & 15)"),
    "q4_0_offset_dropped": ("case BF_Q4_0", "(double)(q - 8)", "(double)(q)"),
    "q8_0_unsigned": ("case BF_Q8_0", "int q = (int8_t)b[2 + e];", "int q = b[2 + e];"),
    "k_high_scale_bits_from_wrong_byte": ("static void scale_min", "((sc[j - 4] >> 6) << 4)",
                                          "((sc[j] >> 6) << 4)"),
    "k_min_high_nibble_swapped": ("static void scale_min", "*m = (sc[j + 4] >> 4)", "*m = (sc[j + 4] & 15)"),
    "k_min_sign": ("case BF_Q4_K", "*w = t1 - t2;", "*w = t1 + t2;"),
    "k_sub_block_order": ("case BF_Q4_K", "int j = 2 * p + hi;", "int j = p + 4 * hi;"),
    "q5_k_fifth_bit_index": ("case BF_Q4_K", "((qh[l] >> j) & 1)", "((qh[l] >> p) & 1)"),
    "q6_k_scale_per_32": ("case BF_Q6_K", "sc[e / 16]", "sc[e / 32]"),
    "q6_k_quarter_nibble": ("case BF_Q6_K", "lo = (t >> 1) ? (lo >> 4) : (lo & 15);",
                            "lo = (t & 1) ? (lo >> 4) : (lo & 15);"),
    "q6_k_offset_dropped": ("case BF_Q6_K", "(double)(q - 32)", "(double)(q)"),
    "f16_bias": ("static double f16_at", "e - 25", "e - 24"),
    "row_stride": ("static void weight", "(n * (K / be) + k / be) * bb", "(n * (K / be) + k / be) * be"),
    "bound_min_term_dropped": ("case BF_Q4_K", "*a = fabs(t1) + fabs(t2);", "*a = fabs(t1 - t2);"),
    "gemv_last_term_dropped": ("void blockref_gemv_rows", "for (int64_t k = 0; k < K; ++k)",
                               "for (int64_t k = 0; k + 1 < K; ++k)"),
}


def _mutant(tmp_path, name):
    anchor, old, new = MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "blockref.c")).read()
    i = src.index(anchor)
    j = src.index(old, i)
    path = tmp_path / f"{name}.c"
    path.write_text(src[:j] + new + src[j + len(old):])
    return blocks.BlockOracle(oracle.build(src=str(path), out=str(tmp_path / f"lib{name}.so")))


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_block_pins_catch_planted_mistakes(tmp_path, name):
    o = _mutant(tmp_path, name)
    caught = []
    for pin in PINS:
        try:
            pin(o)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
