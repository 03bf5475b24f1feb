"""CPU oracle for the int4 decode GEMV (ctypes wrapper around q4ref.c).

TEST INFRASTRUCTURE ONLY.  The product path (the memory_bandwidth_amd package
and its HIP library) never imports this module; only the tests, the smoke
check and the benchmark's CPU-baseline leg do.  The oracle shares no code with
the HIP path.

All functions take numpy arrays in the storage format described in
``workloads`` and return float64 results (GEMVs) or exact float32/uint8
arrays (dequantisation).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4ref.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libq4ref.so")


def build(cflags: tuple[str, ...] = ("-O2",), src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile an oracle source with gcc into a shared library; returns its path."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", *cflags, "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _arr(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    if a is None:
        return None
    assert a.flags.c_contiguous
    return a.ctypes.data


def _check_q4(wq, scales, zeros, N, K, g):
    G = K // g
    if K % g or K % 2:
        raise ValueError("K must be a multiple of g (and of 2)")
    if wq.shape != (N, K // 2) or scales.shape != (N, G) or zeros.shape != (N, (G + 1) // 2):
        raise ValueError(f"bad shapes wq{wq.shape} scales{scales.shape} zeros{zeros.shape} "
                         f"for N={N} K={K} g={g}")


class Oracle:
    """One loaded copy of the oracle library: the default build, or a variant
    compiled from another source by the tests that plant mistakes in it."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.q4ref_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.q4ref_f16_to_f64.restype = ctypes.c_double
        lib.q4ref_dequant.argtypes = [P, P, P, I, I, I, P, P]
        lib.q4ref_gemv_q4_rows.argtypes = [P, P, P, P, I, I, I, I, P, I, P, P]
        lib.q4ref_gemv_q4.argtypes = [P, P, P, P, I, I, I, I, P, P]
        lib.q4ref_gemv_f32_rows.argtypes = [P, P, I, I, I, P, I, P, P]
        lib.q4ref_gemv_f32.argtypes = [P, P, I, I, I, P, P]
        lib.q4ref_sum.argtypes = [P, I, P, P]
        lib.q4ref_quantize.argtypes = [P, P, P, I, I, I, P]
        for f in ("q4ref_dequant", "q4ref_gemv_q4_rows", "q4ref_gemv_q4",
                  "q4ref_gemv_f32_rows", "q4ref_gemv_f32", "q4ref_sum", "q4ref_quantize"):
            getattr(lib, f).restype = None
        self.lib = lib
        self.path = path

    def f16_to_f64(self, bits: int) -> float:
        return self.lib.q4ref_f16_to_f64(bits)

    def dequant(self, wq, scales, zeros, K: int, g: int):
        """Returns (W float32 [N, K], codes uint8 [N, K])."""
        wq, scales, zeros = _arr(wq, np.uint8), _arr(scales, np.uint16), _arr(zeros, np.uint8)
        N = wq.shape[0]
        _check_q4(wq, scales, zeros, N, K, g)
        w = np.empty((N, K), np.float32)
        c = np.empty((N, K), np.uint8)
        self.lib.q4ref_dequant(_ptr(wq), _ptr(scales), _ptr(zeros), N, K, g, _ptr(w), _ptr(c))
        return w, c

    def gemv_q4(self, x, wq, scales, zeros, g: int, rows=None):
        """Returns (y float64 [M, R], bound float64 [M, R]) for the listed rows (default all)."""
        x = _arr(np.atleast_2d(x), np.float32)
        wq, scales, zeros = _arr(wq, np.uint8), _arr(scales, np.uint16), _arr(zeros, np.uint8)
        M, K = x.shape
        N = wq.shape[0]
        _check_q4(wq, scales, zeros, N, K, g)
        if rows is None:
            y = np.empty((M, N), np.float64)
            b = np.empty((M, N), np.float64)
            self.lib.q4ref_gemv_q4(_ptr(x), _ptr(wq), _ptr(scales), _ptr(zeros), M, N, K, g,
                                   _ptr(y), _ptr(b))
            return y, b
        rows = _arr(rows, np.int64)
        if rows.size and (rows.min() < 0 or rows.max() >= N):
            raise IndexError("row index out of range")
        y = np.empty((M, rows.size), np.float64)
        b = np.empty((M, rows.size), np.float64)
        self.lib.q4ref_gemv_q4_rows(_ptr(x), _ptr(wq), _ptr(scales), _ptr(zeros), M, N, K, g,
                                    _ptr(rows), rows.size, _ptr(y), _ptr(b))
        return y, b

    def gemv_f32(self, x, w, rows=None):
        """Dense control.  Returns (y float64 [M, R], bound float64 [M, R])."""
        x = _arr(np.atleast_2d(x), np.float32)
        w = _arr(w, np.float32)
        M, K = x.shape
        N = w.shape[0]
        if w.shape != (N, K):
            raise ValueError("w must be [N, K]")
        if rows is None:
            y = np.empty((M, N), np.float64)
            b = np.empty((M, N), np.float64)
            self.lib.q4ref_gemv_f32(_ptr(x), _ptr(w), M, N, K, _ptr(y), _ptr(b))
            return y, b
        rows = _arr(rows, np.int64)
        if rows.size and (rows.min() < 0 or rows.max() >= N):
            raise IndexError("row index out of range")
        y = np.empty((M, rows.size), np.float64)
        b = np.empty((M, rows.size), np.float64)
        self.lib.q4ref_gemv_f32_rows(_ptr(x), _ptr(w), M, N, K, _ptr(rows), rows.size,
                                     _ptr(y), _ptr(b))
        return y, b

    def buffer_sum(self, buf):
        """Returns (sum, abs-sum) of a float32 buffer in f64."""
        buf = _arr(buf, np.float32).reshape(-1)
        s = ctypes.c_double()
        a = ctypes.c_double()
        self.lib.q4ref_sum(_ptr(buf), buf.size, ctypes.byref(s), ctypes.byref(a))
        return s.value, a.value

    def quantize(self, w, scales, zeros, g: int):
        """Test helper: inverse of dequant for given scales/zeros.  Returns wq uint8 [N, K/2]."""
        w = _arr(w, np.float32)
        scales, zeros = _arr(scales, np.uint16), _arr(zeros, np.uint8)
        N, K = w.shape
        out = np.zeros((N, K // 2), np.uint8)
        self.lib.q4ref_quantize(_ptr(w), _ptr(scales), _ptr(zeros), N, K, g, _ptr(out))
        return out


_default = None


def load() -> Oracle:
    """The default oracle build (compiled on first use when missing)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _default = Oracle(_LIB_PATH)
    return _default


def f16_to_f64(bits: int) -> float:
    return load().f16_to_f64(bits)


def dequant(wq, scales, zeros, K: int, g: int):
    return load().dequant(wq, scales, zeros, K, g)


def gemv_q4(x, wq, scales, zeros, g: int, rows=None):
    return load().gemv_q4(x, wq, scales, zeros, g, rows)


def gemv_f32(x, w, rows=None):
    return load().gemv_f32(x, w, rows)


def buffer_sum(buf):
    return load().buffer_sum(buf)


def quantize(w, scales, zeros, g: int):
    return load().quantize(w, scales, zeros, g)


def gemv_tolerance(bound: np.ndarray) -> np.ndarray:
    """Allowed |y - y_ref| for a GEMV output: 1e-4 * sum|w x| + 1e-6."""
    return 1e-4 * bound + 1e-6


def silu(v) -> np.ndarray:
    """silu(v) = v / (1 + e^-v) in f64 (gerbil "WGSL Kernel Reference",
    section 9 SiLU).  e^-v overflows to inf for v < -709, giving -0."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def swiglu(x, gate, up, g: int, rows=None):
    """SwiGLU combine of two int4 GEMVs of the same x (section 12 Mul: the
    combine is silu(gate) * up).  gate and up are (wq, scales, zeros).
    Returns (y, tol): y = silu(x . Wg^T) * (x . Wu^T) in f64, and the allowed
    |y_gpu - y| per output, propagated from the two GEMV tolerances t_g, t_u:
    |silu'| <= 1.1 everywhere, so the error is at most
    1.1 t_g (|u| + t_u) + |silu(g)| t_u, plus 1e-6 |y| for the rounding of
    the exponential, division and product in fp32."""
    gy, gb = gemv_q4(x, *gate, g, rows)
    uy, ub = gemv_q4(x, *up, g, rows)
    y = silu(gy) * uy
    tg, tu = gemv_tolerance(gb), gemv_tolerance(ub)
    tol = 1.1 * tg * (np.abs(uy) + tu) + np.abs(silu(gy)) * tu + 1e-6 * np.abs(y)
    return y, tol
