"""CPU oracle for the 2-bit corpus scan (ctypes wrapper around scanref.c).

TEST INFRASTRUCTURE ONLY.  The product path never imports this module; only
the tests, the smoke check and the benchmark's CPU-baseline leg do.  It shares
no code with the HIP path.

codes: uint32 [V, D/16], 16 two-bit codes per word, dimension 16w + i in bits
2i, 2i+1 of word w.  lut: float32 [Q, D, 4].  Returns float64 scores [R, Q] and
the float64 bound sum |lut term| the tolerance is built from.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from oracle import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "scanref.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libscanref.so")


def build() -> str:
    return _build(src=_SRC, out=_LIB_PATH)


class ScanOracle:
    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P, I = ctypes.c_void_p, ctypes.c_int64
        lib.scanref_rows.argtypes = [P, I, I, P, I, P, I, P, P]
        lib.scanref_rows.restype = None
        self.lib = lib

    def scan(self, codes, lut, rows=None):
        codes = np.ascontiguousarray(codes, dtype=np.uint32)
        lut = np.ascontiguousarray(lut, dtype=np.float32)
        if codes.ndim != 2 or lut.ndim != 3 or lut.shape[2] != 4:
            raise ValueError("codes must be [V, D/16] and lut [Q, D, 4]")
        V, W = codes.shape
        Q, D, _ = lut.shape
        if D != 16 * W:
            raise ValueError(f"lut has D = {D}, codes hold {16 * W} dimensions")
        rows = np.arange(V, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
        if rows.size and (rows.min() < 0 or rows.max() >= V):
            raise IndexError("vector index out of range")
        s = np.empty((rows.size, Q), np.float64)
        b = np.empty((rows.size, Q), np.float64)
        self.lib.scanref_rows(codes.ctypes.data, V, D, lut.ctypes.data, Q, rows.ctypes.data,
                              rows.size, s.ctypes.data, b.ctypes.data)
        return s, b


_default = None


def load() -> ScanOracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _default = ScanOracle(_LIB_PATH)
    return _default


def scan(codes, lut, rows=None):
    return load().scan(codes, lut, rows)


def scan_tolerance(bound: np.ndarray) -> np.ndarray:
    """Allowed |score - score_ref|: 1e-4 * sum |term| + 1e-6, the GEMV rule."""
    return 1e-4 * bound + 1e-6
