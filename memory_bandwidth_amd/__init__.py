"""Thin Python binding of libq4gemv.so (the MI355X int4 decode-GEMV library).

Every function has the name of the C entry point it calls and only marshals
arguments: it checks dtypes, shapes, contiguity and device, passes raw device
pointers and torch's current HIP stream, and raises Q4Error on a non-zero
status.  All arithmetic runs in the library's HIP kernels; there is no other
implementation here.  Importing this module without the built library works
(so CPU-only tooling can inspect it), but every call then raises.

Storage format (see include/q4gemv.h): x float32 [M, K]; wq uint8 [N, K/2]
(two codes per byte, low nibble = even k); scales float16 or uint16 [N, K/g]
(binary16 bits); zeros uint8 [N, ceil(K/g / 2)] (low nibble = even group).
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4gemv.so")

Q4_OK, Q4_EINVAL, Q4_ENULL, Q4_EALIGN, Q4_EDEVICE, Q4_ELAUNCH = 0, -1, -2, -3, -4, -5

# Exported C symbols, in the order include/q4gemv.h, include/q4blocks.h and
# include/q4scan.h declare them.
EXPORTS = ("gemv_q4", "gemv_q4_ws", "gemv_q4_workspace_size", "gemv_q4_static", "gemv_q4_swiglu", "gemv_f32", "dequant_q4", "read_reduce",
           "read_reduce_passes", "copy_vec4", "write_fill",
           "gemv_q4_geometry", "gemv_q4_path", "q4_strerror", "q4_abi_version",
           "gemv_q4_set_geometry", "gemv_q4_clear_geometry",
           "block_geometry", "gemv_block", "dequant_block", "gemv_block_set_config",
           "gemv_block_config", "scan2", "scan2_set_config", "scan2_config")

# Block formats of include/q4blocks.h.
BLK_Q4_0, BLK_Q8_0, BLK_Q4_K, BLK_Q5_K, BLK_Q6_K = 1, 2, 3, 4, 5
BLOCK_FORMATS = {"q4_0": BLK_Q4_0, "q8_0": BLK_Q8_0, "q4_k": BLK_Q4_K, "q5_k": BLK_Q5_K,
                 "q6_k": BLK_Q6_K}

Q4_PATH_FMA, Q4_PATH_INTEGER = 0, 1

_lib = None


class Q4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {strerror(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library {LIB_PATH} is not built; run "
                           "`python -m memory_bandwidth_amd.build` first")
    L = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.gemv_q4.argtypes = [P, P, P, P, P, I, I, I, I, P]
    L.gemv_q4_ws.argtypes = [P, P, P, P, P, I, I, I, I, P, Z, P]
    L.gemv_q4_workspace_size.argtypes = [I, I, I, I, ctypes.POINTER(Z)]
    L.gemv_q4_static.argtypes = [P, P, P, P, P, I, I, I, I, P]
    L.gemv_q4_swiglu.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, P]
    L.gemv_f32.argtypes = [P, P, P, I, I, I, P]
    L.dequant_q4.argtypes = [P, P, P, P, P, I, I, I, P]
    L.read_reduce.argtypes = [P, Z, P, I, P]
    L.read_reduce_passes.argtypes = [P, Z, I, P, I, P]
    L.copy_vec4.argtypes = [P, P, Z, I, I, P]
    L.write_fill.argtypes = [P, Z, ctypes.c_float, I, P]
    IP = ctypes.POINTER(ctypes.c_int)
    L.gemv_q4_geometry.argtypes = [I, I, I, I, IP, IP, IP, IP, IP, IP]
    L.gemv_q4_path.argtypes = [I, I, I, I]
    L.gemv_q4_set_geometry.argtypes = [I, I, I, I, I, I, I]
    L.gemv_q4_clear_geometry.argtypes = []
    L.block_geometry.argtypes = [I, IP, IP]
    L.gemv_block.argtypes = [I, P, P, P, I, I, I, P]
    L.dequant_block.argtypes = [I, P, P, I, I, P]
    L.gemv_block_set_config.argtypes = [I, I, I, I]
    L.gemv_block_config.argtypes = [I, IP, IP, IP]
    L.scan2.argtypes = [P, P, P, I, I, I, P]
    L.scan2_set_config.argtypes = [I, I, I, I]
    L.scan2_config.argtypes = [IP, IP, IP, IP]
    L.q4_strerror.argtypes = [I]
    L.q4_strerror.restype = ctypes.c_char_p
    L.q4_abi_version.argtypes = []
    for f in ("gemv_q4", "gemv_q4_ws", "gemv_q4_workspace_size", "gemv_q4_static", "gemv_q4_swiglu", "gemv_f32", "dequant_q4", "read_reduce",
              "read_reduce_passes", "copy_vec4", "write_fill", "gemv_q4_geometry", "gemv_q4_path", "q4_abi_version",
              "gemv_q4_set_geometry", "gemv_q4_clear_geometry", "block_geometry", "gemv_block",
              "dequant_block", "gemv_block_set_config", "gemv_block_config", "scan2",
              "scan2_set_config", "scan2_config"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().q4_strerror(status).decode()


def _check(fn: str, status: int) -> None:
    if status != Q4_OK:
        raise Q4Error(fn, status)


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t: torch.Tensor, name: str, dtypes, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _q4_operands(x: torch.Tensor, wq: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                 group_size: int, N: int | None = None):
    """Checks one int4 matrix against x; returns (M, N, K, g)."""
    _need(x, "x", (torch.float32,))
    dev = x.device
    _need(wq, "wq", (torch.uint8,), dev)
    _need(scales, "scales", (torch.float16, torch.uint16, torch.int16), dev)
    _need(zeros, "zeros", (torch.uint8,), dev)
    if x.dim() != 2 or wq.dim() != 2:
        raise ValueError("x must be [M, K] and wq [N, K/2]")
    M, K = x.shape
    n = wq.shape[0]
    g = int(group_size)
    G = K // g if g else 0
    if (wq.shape[1] * 2 != K or tuple(scales.shape) != (n, G) or tuple(zeros.shape) != (n, (G + 1) // 2)
            or (N is not None and n != N)):
        raise ValueError(f"shape mismatch: x{tuple(x.shape)} wq{tuple(wq.shape)} "
                         f"scales{tuple(scales.shape)} zeros{tuple(zeros.shape)} g={g}")
    return M, n, K, g


def _out(out: torch.Tensor | None, M: int, N: int, dev: torch.device) -> torch.Tensor:
    if out is None:
        return torch.empty((M, N), dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), dev)
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    return out


def gemv_q4_workspace_size(M: int, N: int, K: int, group_size: int) -> int:
    """Workspace bytes with which gemv_q4_ws may split K over workgroups (0: none needed)."""
    n = ctypes.c_size_t()
    _check("gemv_q4_workspace_size", lib().gemv_q4_workspace_size(M, N, K, group_size, ctypes.byref(n)))
    return n.value


def gemv_q4(x: torch.Tensor, wq: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
            group_size: int, out: torch.Tensor | None = None,
            workspace: torch.Tensor | bool | None = None) -> torch.Tensor:
    """y[M, N] = x[M, K] . dequant(W_q[N, K])^T on the current stream.

    workspace: None takes one from torch's allocator when the shape can use
    it (gemv_q4_ws); a uint8 tensor on x's device is used as given; False
    calls gemv_q4 without one."""
    M, N, K, g = _q4_operands(x, wq, scales, zeros, group_size)
    out = _out(out, M, N, x.device)
    if workspace is False:
        _check("gemv_q4", lib().gemv_q4(_ptr(x), _ptr(wq), _ptr(scales), _ptr(zeros), _ptr(out),
                                        M, N, K, g, _stream(x.device)))
        return out
    if workspace is None or workspace is True:
        n = gemv_q4_workspace_size(M, N, K, g)
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device) if n else None
    else:
        _need(workspace, "workspace", (torch.uint8,), x.device)
    wp, wn = (_ptr(workspace), workspace.numel()) if workspace is not None else (None, 0)
    _check("gemv_q4_ws", lib().gemv_q4_ws(_ptr(x), _ptr(wq), _ptr(scales), _ptr(zeros), _ptr(out),
                                          M, N, K, g, wp, wn, _stream(x.device)))
    return out


def gemv_q4_swiglu(x: torch.Tensor, gate: tuple, up: tuple, group_size: int,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """y = silu(x . Wg^T) * (x . Wu^T); gate and up are (wq, scales, zeros)."""
    M, N, K, g = _q4_operands(x, *gate, group_size)
    _q4_operands(x, *up, group_size, N=N)
    out = _out(out, M, N, x.device)
    (wg, sg, zg), (wu, su, zu) = gate, up
    _check("gemv_q4_swiglu", lib().gemv_q4_swiglu(
        _ptr(x), _ptr(wg), _ptr(sg), _ptr(zg), _ptr(wu), _ptr(su), _ptr(zu), _ptr(out),
        M, N, K, g, _stream(x.device)))
    return out


def gemv_f32(x: torch.Tensor, w: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Dense control: y[M, N] = x[M, K] . w[N, K]^T on the current stream."""
    _need(x, "x", (torch.float32,))
    dev = x.device
    _need(w, "w", (torch.float32,), dev)
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x must be [M, K] and w [N, K]")
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=dev)
    else:
        _need(out, "out", (torch.float32,), dev)
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be [M, N]")
    _check("gemv_f32", lib().gemv_f32(_ptr(x), _ptr(w), _ptr(out), M, N, K, _stream(dev)))
    return out


def dequant_q4(wq: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor, group_size: int,
               want_weights: bool = True, want_codes: bool = True):
    """Returns (W float32 [N, K] or None, codes uint8 [N, K] or None)."""
    _need(wq, "wq", (torch.uint8,))
    dev = wq.device
    _need(scales, "scales", (torch.float16, torch.uint16, torch.int16), dev)
    _need(zeros, "zeros", (torch.uint8,), dev)
    N, K = wq.shape[0], wq.shape[1] * 2
    g = int(group_size)
    G = K // g if g else 0
    if tuple(scales.shape) != (N, G) or tuple(zeros.shape) != (N, (G + 1) // 2):
        raise ValueError("scales/zeros shape mismatch")
    w = torch.empty((N, K), dtype=torch.float32, device=dev) if want_weights else None
    c = torch.empty((N, K), dtype=torch.uint8, device=dev) if want_codes else None
    _check("dequant_q4", lib().dequant_q4(_ptr(wq), _ptr(scales), _ptr(zeros), _ptr(w), _ptr(c),
                                          N, K, g, _stream(dev)))
    return w, c


def _partials(buf: torch.Tensor, n_partials: int, partials: torch.Tensor | None) -> torch.Tensor:
    _need(buf, "buf", (torch.float32,))
    if partials is None:
        return torch.empty(n_partials, dtype=torch.float32, device=buf.device)
    _need(partials, "partials", (torch.float32,), buf.device)
    if partials.numel() < n_partials:
        raise ValueError("partials too small")
    return partials


def read_reduce(buf: torch.Tensor, n_partials: int, partials: torch.Tensor | None = None) -> torch.Tensor:
    """Launches the streaming read probe (non-temporal loads); returns the
    per-workgroup partial sums (add them for the total)."""
    partials = _partials(buf, n_partials, partials)
    _check("read_reduce", lib().read_reduce(_ptr(buf), buf.numel(), _ptr(partials), n_partials,
                                            _stream(buf.device)))
    return partials


def read_reduce_passes(buf: torch.Tensor, n_partials: int, passes: int,
                       partials: torch.Tensor | None = None) -> torch.Tensor:
    """The read probe walking buf `passes` times with plain loads (so that a
    buffer that fits a cache is re-read from it); per-workgroup partial sums."""
    partials = _partials(buf, n_partials, partials)
    _check("read_reduce_passes", lib().read_reduce_passes(
        _ptr(buf), buf.numel(), passes, _ptr(partials), n_partials, _stream(buf.device)))
    return partials


def copy_vec4(src: torch.Tensor, dst: torch.Tensor | None = None, passes: int = 1,
              n_blocks: int = 0) -> torch.Tensor:
    """Copies src into dst (a new tensor if None) with the copy probe."""
    _need(src, "src", (torch.float32,))
    if dst is None:
        dst = torch.empty_like(src)
    else:
        _need(dst, "dst", (torch.float32,), src.device)
        if dst.numel() != src.numel():
            raise ValueError("dst and src differ in size")
    _check("copy_vec4", lib().copy_vec4(_ptr(src), _ptr(dst), src.numel(), passes, n_blocks,
                                        _stream(src.device)))
    return dst


def write_fill(buf: torch.Tensor, value: float, n_blocks: int = 0) -> torch.Tensor:
    """Fills buf with value using the write probe."""
    _need(buf, "buf", (torch.float32,))
    _check("write_fill", lib().write_fill(_ptr(buf), buf.numel(), float(value), n_blocks,
                                          _stream(buf.device)))
    return buf


def gemv_q4_geometry(M: int, N: int, K: int, group_size: int) -> dict:
    """Launch geometry gemv_q4 picks for a shape (host-only, needs no GPU)."""
    vals = [ctypes.c_int() for _ in range(6)]
    _check("gemv_q4_geometry", lib().gemv_q4_geometry(M, N, K, group_size,
                                                      *[ctypes.byref(v) for v in vals]))
    keys = ("grid", "block", "rows_per_wave", "lanes_per_row", "ksplit", "segments")
    return {k: v.value for k, v in zip(keys, vals)}


def gemv_q4_path(M: int, N: int, K: int, group_size: int) -> int:
    """Q4_PATH_FMA or Q4_PATH_INTEGER: the arithmetic path gemv_q4 takes (host-only)."""
    r = lib().gemv_q4_path(M, N, K, group_size)
    if r < 0:
        raise Q4Error("gemv_q4_path", r)
    return r


def abi_version() -> int:
    return lib().q4_abi_version()


def gemv_q4_set_geometry(M: int, N: int, K: int, group_size: int, path: int, waves: int = 0,
                         ksplit: int = 0) -> None:
    """Fix gemv_q4's geometry for one exact shape (host-only); raises Q4Error
    when the kernels cannot run that combination."""
    _check("gemv_q4_set_geometry", lib().gemv_q4_set_geometry(M, N, K, group_size, path, waves, ksplit))


def gemv_q4_clear_geometry() -> None:
    """Forget every geometry fixed by gemv_q4_set_geometry."""
    _check("gemv_q4_clear_geometry", lib().gemv_q4_clear_geometry())


# ---------------------------------------------------------------- block formats

def _fmt(fmt) -> int:
    if isinstance(fmt, str):
        if fmt not in BLOCK_FORMATS:
            raise ValueError(f"unknown block format {fmt!r}")
        return BLOCK_FORMATS[fmt]
    return int(fmt)


def block_geometry(fmt) -> tuple[int, int]:
    """(elements, bytes) of one block of the format (host-only)."""
    e, b = ctypes.c_int(), ctypes.c_int()
    _check("block_geometry", lib().block_geometry(_fmt(fmt), ctypes.byref(e), ctypes.byref(b)))
    return e.value, b.value


def _block_matrix(fmt, w: torch.Tensor, K: int, dev=None) -> tuple[int, int]:
    _need(w, "w", (torch.uint8,), dev)
    e, b = block_geometry(fmt)
    if w.dim() != 2 or K % e or w.shape[1] != K // e * b:
        raise ValueError(f"w must be [N, K / {e} * {b}] bytes for K = {K}, got {tuple(w.shape)}")
    return w.shape[0], K // e * b


def gemv_block(fmt, x: torch.Tensor, w: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """y[1, N] = x[1, K] . W^T for a block-format matrix w uint8 [N, row_bytes]."""
    _need(x, "x", (torch.float32,))
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    N, _ = _block_matrix(fmt, w, K, x.device)
    out = _out(out, M, N, x.device)
    _check("gemv_block", lib().gemv_block(_fmt(fmt), _ptr(x), _ptr(w), _ptr(out), M, N, K,
                                          _stream(x.device)))
    return out


def dequant_block(fmt, w: torch.Tensor, K: int) -> torch.Tensor:
    """W float32 [N, K], bit-exact, from a block-format matrix."""
    N, _ = _block_matrix(fmt, w, K)
    out = torch.empty((N, K), dtype=torch.float32, device=w.device)
    _check("dequant_block", lib().dequant_block(_fmt(fmt), _ptr(w), _ptr(out), N, K,
                                                _stream(w.device)))
    return out


def gemv_block_set_config(fmt, rows_per_lane: int = 0, waves_per_group: int = 0,
                          groups_per_cu: int = 0) -> None:
    """Row slots per lane (1, 2, 4), wavefronts per workgroup (4, 8) and
    workgroups per CU (0 = one per row block) of gemv_block for one format;
    all zero restores the default (host-only)."""
    _check("gemv_block_set_config", lib().gemv_block_set_config(_fmt(fmt), rows_per_lane,
                                                                waves_per_group, groups_per_cu))


def gemv_block_config(fmt) -> tuple[int, int, int]:
    v = [ctypes.c_int() for _ in range(3)]
    _check("gemv_block_config", lib().gemv_block_config(_fmt(fmt), *[ctypes.byref(t) for t in v]))
    return tuple(t.value for t in v)


# ---------------------------------------------------------------- 2-bit scan

def scan2(codes: torch.Tensor, lut: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """scores[V, Q] = sum_d lut[q, d, code(v, d)] for codes uint32 (or int32)
    [V, D/16] and lut float32 [Q, D, 4]."""
    _need(codes, "codes", (torch.int32, torch.uint32) if hasattr(torch, "uint32") else (torch.int32,))
    dev = codes.device
    _need(lut, "lut", (torch.float32,), dev)
    if codes.dim() != 2 or lut.dim() != 3 or lut.shape[2] != 4 or lut.shape[1] != 16 * codes.shape[1]:
        raise ValueError(f"codes must be [V, D/16] and lut [Q, D, 4]: got {tuple(codes.shape)}, "
                         f"{tuple(lut.shape)}")
    V, Q, D = codes.shape[0], lut.shape[0], lut.shape[1]
    out = _out(out, V, Q, dev)
    _check("scan2", lib().scan2(_ptr(codes), _ptr(lut), _ptr(out), V, D, Q, _stream(dev)))
    return out


def scan2_set_config(lut_in_lds: int = 0, vectors_per_thread: int = 0,
                     threads_per_group: int = 0, threads_per_vector: int = 0) -> None:
    """The scan's knobs: table in LDS (1) or memory (0), vectors per thread
    (1, 2), threads per workgroup (64, 256, 1024), threads per vector (1, 2,
    4, 8; an upper bound); all zero restores the default (host-only)."""
    _check("scan2_set_config", lib().scan2_set_config(lut_in_lds, vectors_per_thread,
                                                      threads_per_group, threads_per_vector))


def scan2_config() -> tuple[int, int, int, int]:
    v = [ctypes.c_int() for _ in range(4)]
    _check("scan2_config", lib().scan2_config(*[ctypes.byref(t) for t in v]))
    return tuple(t.value for t in v)
