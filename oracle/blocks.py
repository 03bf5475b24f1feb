"""CPU oracle for the block-format decode GEMV (ctypes wrapper around blockref.c).

TEST INFRASTRUCTURE ONLY.  The product path never imports this module; only
the tests, the smoke check and the benchmark's CPU-baseline leg do.  It shares
no code with the HIP path.

A matrix in a block format is a uint8 array [N, (K / elems) * bytes]: each row
is its K / elems blocks one after another.  x is float32 [M, K].  GEMVs return
float64 results and the float64 bound the tolerance is built from.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from oracle import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "blockref.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libblockref.so")

# Format codes (shared by value with the library's BLK_* constants; the two
# sides agree through the tests, not through a common header).
Q4_0, Q8_0, Q4_K, Q5_K, Q6_K = 1, 2, 3, 4, 5
NAMES = {Q4_0: "q4_0", Q8_0: "q8_0", Q4_K: "q4_k", Q5_K: "q5_k", Q6_K: "q6_k"}


def build() -> str:
    return _build(src=_SRC, out=_LIB_PATH)


class BlockOracle:
    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P, I = ctypes.c_void_p, ctypes.c_int64
        lib.blockref_geometry.argtypes = [ctypes.c_int, ctypes.POINTER(I), ctypes.POINTER(I)]
        lib.blockref_geometry.restype = ctypes.c_int
        lib.blockref_dequant.argtypes = [ctypes.c_int, P, I, I, P]
        lib.blockref_dequant.restype = None
        lib.blockref_gemv_rows.argtypes = [ctypes.c_int, P, P, I, I, I, P, I, P, P]
        lib.blockref_gemv_rows.restype = None
        self.lib = lib

    def geometry(self, fmt: int) -> tuple[int, int]:
        e, b = ctypes.c_int64(), ctypes.c_int64()
        if not self.lib.blockref_geometry(fmt, ctypes.byref(e), ctypes.byref(b)):
            raise ValueError(f"unknown block format {fmt}")
        return e.value, b.value

    def row_bytes(self, fmt: int, K: int) -> int:
        e, b = self.geometry(fmt)
        if K % e:
            raise ValueError(f"K = {K} is not a multiple of the block size {e}")
        return K // e * b

    def _check(self, fmt, w, K):
        w = np.ascontiguousarray(w, dtype=np.uint8)
        if w.ndim != 2 or w.shape[1] != self.row_bytes(fmt, K):
            raise ValueError(f"w must be [N, {self.row_bytes(fmt, K)}] bytes, got {w.shape}")
        return w

    def dequant(self, fmt: int, w, K: int) -> np.ndarray:
        """float32 [N, K]: every weight rounded once from its exact value."""
        w = self._check(fmt, w, K)
        N = w.shape[0]
        out = np.empty((N, K), np.float32)
        self.lib.blockref_dequant(fmt, w.ctypes.data, N, K, out.ctypes.data)
        return out

    def gemv(self, fmt: int, x, w, rows=None):
        """(y float64 [M, R], bound float64 [M, R]) for the listed rows (default all)."""
        x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
        M, K = x.shape
        w = self._check(fmt, w, K)
        N = w.shape[0]
        rows = np.arange(N, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
        if rows.size and (rows.min() < 0 or rows.max() >= N):
            raise IndexError("row index out of range")
        y = np.empty((M, rows.size), np.float64)
        b = np.empty((M, rows.size), np.float64)
        self.lib.blockref_gemv_rows(fmt, x.ctypes.data, w.ctypes.data, M, N, K,
                                    rows.ctypes.data, rows.size, y.ctypes.data, b.ctypes.data)
        return y, b


_default = None


def load() -> BlockOracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _default = BlockOracle(_LIB_PATH)
    return _default


def geometry(fmt: int) -> tuple[int, int]:
    return load().geometry(fmt)


def row_bytes(fmt: int, K: int) -> int:
    return load().row_bytes(fmt, K)


def dequant(fmt: int, w, K: int) -> np.ndarray:
    return load().dequant(fmt, w, K)


def gemv(fmt: int, x, w, rows=None):
    return load().gemv(fmt, x, w, rows)


def gemv_tolerance(bound: np.ndarray) -> np.ndarray:
    """Allowed |y - y_ref|: 1e-4 * bound + 1e-6, as for the int4 GEMV."""
    return 1e-4 * bound + 1e-6
