"""Seeded synthetic inputs for the int4 decode GEMV and its probes.

This module draws random numbers and lays them out in the storage format; it
holds none of the GEMV's arithmetic (no unpacking, no dequantisation, no dot
products).  Both the HIP path and the oracle take its arrays as inputs.

Storage format (gerbil "WGSL Kernel Reference", section 3 MatMulInt4,
"INT4 Packing" and "Dequantization", read N-major as the decode GEMV
y = x . dequant(W_q)^T):

  wq      uint8  [N, K/2]      two 4-bit codes per byte along K,
                                low nibble = even k, high nibble = odd k
  scales  uint16 [N, G]        IEEE binary16 bit patterns, G = K / g
  zeros   uint8  [N, ceil(G/2)] two 4-bit zero points per byte along the
                                group axis, low nibble = even group
  x       float32 [M, K]       row-major activations

Random bytes that are uniform over 0..255 carry two independent codes that
are uniform over 0..15, so the packed arrays are drawn byte-wise.
"""

from __future__ import annotations

import dataclasses
import numpy as np

# Per-tensor stream ids: every tensor gets its own SeedSequence child so that
# changing one shape never shifts another tensor's values.
_STREAM_X, _STREAM_WQ, _STREAM_S, _STREAM_Z = 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Q4Shape:
    """One GEMV shape: y[M, N] = x[M, K] . dequant(W_q[N, K])^T."""

    M: int
    N: int
    K: int
    g: int
    s_lo: float
    s_hi: float
    label: str = ""

    @property
    def G(self) -> int:
        return self.K // self.g

    @property
    def ZB(self) -> int:
        return (self.G + 1) // 2


def q4_weight_bytes(N: int, K: int, g: int) -> int:
    """Algorithmic bytes one q4 GEMV must read: packed codes + fp16 scales + packed zeros.

    Counts weight-side bytes only, as the cera wgpu_gemv_bench.rs byte
    accounting does (block bytes, no activations); x and y are reported apart.
    """
    G = K // g
    return N * (K // 2) + 2 * N * G + N * ((G + 1) // 2)


def f32_weight_bytes(N: int, K: int) -> int:
    return 4 * N * K


# The five workloads.  Value distributions: codes and zeros uniform over
# 0..15, scales uniform in [s_lo, s_hi] rounded to binary16, x ~ N(0, 1).
SMALL_896 = Q4Shape(1, 896, 896, 32, 0.005, 0.02, "single 896x896 g32")
DECODER_LAYER = (
    Q4Shape(1, 896, 896, 32, 0.005, 0.02, "q_proj"),
    Q4Shape(1, 128, 896, 32, 0.005, 0.02, "k_proj"),
    Q4Shape(1, 128, 896, 32, 0.005, 0.02, "v_proj"),
    Q4Shape(1, 896, 896, 32, 0.005, 0.02, "o_proj"),
    Q4Shape(1, 4864, 896, 32, 0.005, 0.02, "gate_proj"),
    Q4Shape(1, 4864, 896, 32, 0.005, 0.02, "up_proj"),
    Q4Shape(1, 896, 4864, 32, 0.005, 0.02, "down_proj"),
)
LM_HEAD = Q4Shape(1, 151936, 896, 32, 0.005, 0.02, "lm_head 896->151936 g32")


def ffn_8b(M: int) -> tuple[Q4Shape, Q4Shape]:
    return (
        Q4Shape(M, 14336, 4096, 128, 0.002, 0.01, f"ffn up 4096->14336 g128 M={M}"),
        Q4Shape(M, 4096, 14336, 128, 0.002, 0.01, f"ffn down 14336->4096 g128 M={M}"),
    )


STREAM_SHAPE = Q4Shape(1, 14336, 4096, 128, 0.002, 0.01, "stream 4096x14336 g128")
STREAM_MATRICES = 32          # distinct q4 matrices cycled (976,224,256 B > L2 + MALL)
STREAM_F32_MATRICES = 4       # distinct f32 control matrices cycled (939,524,096 B)
PROBE_BYTES = 2 * 1024**3     # read_reduce buffer for the measured HBM roofline


def workload_seed(index: int) -> int:
    return 0x5EED0000 + index


def _rng(seed: int, stream: int, index: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream, index]))


def make_x(seed: int, M: int, K: int, index: int = 0) -> np.ndarray:
    """x[M, K] float32, standard normal, one independent row per token."""
    return _rng(seed, _STREAM_X, index).standard_normal((M, K), dtype=np.float32)


def make_q4_weights(seed: int, N: int, K: int, g: int, s_lo: float, s_hi: float,
                    index: int = 0) -> dict[str, np.ndarray]:
    """Packed codes, fp16 scale bits and packed zero points for one matrix."""
    if K % g or g not in (32, 128):
        raise ValueError(f"need K % g == 0 and g in (32, 128), got K={K} g={g}")
    G = K // g
    ZB = (G + 1) // 2
    wq = _rng(seed, _STREAM_WQ, index).integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = _rng(seed, _STREAM_S, index).uniform(s_lo, s_hi, size=(N, G))
    scales = s.astype(np.float16).view(np.uint16)          # round to nearest even
    zeros = _rng(seed, _STREAM_Z, index).integers(0, 256, size=(N, ZB), dtype=np.uint8)
    if G % 2:
        zeros[:, -1] &= 0x0F                                # unused high nibble
    return {"wq": wq, "scales": scales, "zeros": zeros}


def make_q4_problem(seed: int, shape: Q4Shape, index: int = 0) -> dict[str, np.ndarray]:
    d = make_q4_weights(seed, shape.N, shape.K, shape.g, shape.s_lo, shape.s_hi, index)
    d["x"] = make_x(seed, shape.M, shape.K, index)
    return d


def fuse_rows(*mats: dict) -> dict:
    """Matrices of the same K and group size stored as one: their rows one
    after another (codes, scales and zero points alike), so one GEMV of the
    result computes all of them (q, k and v of a decoder layer as one
    [N_q + N_k + N_v, K] matrix).  Layout only."""
    return {k: np.concatenate([m[k] for m in mats], axis=0) for k in ("wq", "scales", "zeros")}


def make_exact_problem(seed: int, M: int, N: int, K: int, g: int,
                       index: int = 0) -> dict[str, np.ndarray]:
    """Inputs on which fp32 accumulation is exact in any order.

    Scales are powers of two 2^-e with e in 6..10 (exact in binary16) and x
    holds integers in [-2, 2].  Every product (q - z) * s * x is then a
    multiple of 2^-10 of magnitude at most 15 * 2 * 2^-6, so any partial sum
    over at most K terms is a multiple of 2^-10 below 0.47 * K, which fp32
    represents exactly while 0.47 * K < 2^14, i.e. for K <= 34952.
    """
    if K > 34952:
        raise ValueError("exactness argument needs K <= 34952")
    d = make_q4_weights(seed, N, K, g, 0.01, 0.02, index)
    e = _rng(seed, 11, index).integers(6, 11, size=d["scales"].shape)
    d["scales"] = np.ldexp(1.0, -e).astype(np.float16).view(np.uint16)
    d["x"] = _rng(seed, 12, index).integers(-2, 3, size=(M, K)).astype(np.float32)
    return d


# Block formats named on the cera page (wgpu_gemv_bench, the block-geometry
# table): format code, elements per block, bytes per block, and the byte
# offsets of the binary16 fields that scale a block (layout only).
BLOCK_FORMATS = {
    "q4_0": (1, 32, 18, (0,)),
    "q8_0": (2, 32, 34, (0,)),
    "q4_k": (3, 256, 144, (0, 2)),
    "q5_k": (4, 256, 176, (0, 2)),
    "q6_k": (5, 256, 210, (208,)),
}
_STREAM_BLK, _STREAM_BLK_S = 31, 32

# The cera page's decode-GEMV shapes (output rows, K), and the stream shape.
BLOCK_SHAPES = (
    (2816, 1024, "ffn gate/up"),
    (1024, 2816, "ffn down"),
    (1024, 1024, "attn qkv/out"),
    (65536, 1024, "lm head"),
)


def block_row_bytes(fmt: str, K: int) -> int:
    _, e, b, _ = BLOCK_FORMATS[fmt]
    if K % e:
        raise ValueError(f"K = {K} is not a multiple of the {fmt} block size {e}")
    return K // e * b


def make_block_weights(seed: int, fmt: str, N: int, K: int, s_lo: float = 0.002,
                       s_hi: float = 0.01, index: int = 0) -> np.ndarray:
    """One [N, K] matrix in a block format: uint8 [N, (K / elems) * bytes].

    Every byte is uniform over 0..255 (codes, packed sub-block scales and
    mins, int8 values), except the binary16 fields that scale a block, which
    are uniform in [s_lo, s_hi] rounded to binary16, so that no block holds an
    infinity or a NaN.  (The cera page keeps every byte in 0x30..0x37 for the
    same reason; uniform bytes exercise every code.)
    """
    _, e, b, f16_at = BLOCK_FORMATS[fmt]
    rb = block_row_bytes(fmt, K)
    w = _rng(seed, _STREAM_BLK, index).integers(0, 256, size=(N, K // e, b), dtype=np.uint8)
    s = _rng(seed, _STREAM_BLK_S, index).uniform(s_lo, s_hi, size=(N, K // e, len(f16_at)))
    sb = s.astype(np.float16).view(np.uint8).reshape(N, K // e, len(f16_at), 2)
    for i, off in enumerate(f16_at):
        w[:, :, off:off + 2] = sb[:, :, i, :]
    return w.reshape(N, rb)


# The 2-bit corpus scan of the Refractometer page: 65,536 vectors x 8
# queries.  D is not on the page; 768 is the EmbeddingGemma embedding width.
SCAN_VECTORS, SCAN_QUERIES, SCAN_DIM = 65536, 8, 768
_STREAM_SCAN_C, _STREAM_SCAN_Q, _STREAM_SCAN_L = 41, 42, 43


def make_scan_codes(seed: int, V: int, D: int, index: int = 0) -> np.ndarray:
    """codes uint32 [V, D/16]: every 2-bit code uniform over 0..3."""
    if D % 16:
        raise ValueError("D must be a multiple of 16")
    return _rng(seed, _STREAM_SCAN_C, index).integers(0, 2**32, size=(V, D // 16), dtype=np.uint32)


def make_scan_lut(seed: int, Q: int, D: int, index: int = 0) -> np.ndarray:
    """lut float32 [Q, D, 4]: entry (q, d, c) = query[q, d] * level[d, c], the
    table an asymmetric-distance scan builds from each query (query ~ N(0, 1))
    and a per-dimension 2-bit codebook (four sorted levels, N(0, 1) draws)."""
    query = _rng(seed, _STREAM_SCAN_Q, index).standard_normal((Q, D))
    level = np.sort(_rng(seed, _STREAM_SCAN_L, index).standard_normal((D, 4)), axis=1)
    return (query[:, :, None] * level[None, :, :]).astype(np.float32)


def make_probe_buffer(n_floats: int, seed: int = 0x5EED0004) -> np.ndarray:
    """A float32 buffer for the read probe, values uniform in [0, 1)."""
    return _rng(seed, 21, 0).random(n_floats, dtype=np.float32)
