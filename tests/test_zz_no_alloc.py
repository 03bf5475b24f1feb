"""gemv_q4_static (the entry point that allocates nothing: its workspace is
a static device array) against gemv_q4_ws with a caller workspace, through
the C ABI: two calls in a row, the second smaller, each bit-identical to
gemv_q4_ws and within the GEMV bound of the oracle."""
import ctypes

import numpy as np
import pytest

import memory_bandwidth_amd as q4
import oracle
import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CALLS = [(8, 4096, 14336, 128), (4, 300, 14336, 128), (2, 64, 2048, 32)]


def _problem(M, N, K, g, seed):
    s = wl.Q4Shape(M, N, K, g, 0.002, 0.02)
    d = wl.make_q4_problem(seed, s)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda:0") for k, v in d.items()}
    return d, t


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def test_static_workspace_matches_caller_workspace():
    L = q4.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i, (M, N, K, g) in enumerate(CALLS):
        d, t = _problem(M, N, K, g, 900 + i)
        print(f"gemv_q4_static call {i}: M{M} N{N} K{K} g{g}", flush=True)
        need = q4.gemv_q4_workspace_size(M, N, K, g)
        assert need <= 512 * 1024
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda:0")
        y_ws = torch.full((M, N), float("nan"), device="cuda:0")
        y_st = torch.full((M, N), float("nan"), device="cuda:0")
        args = (_ptr(t["x"]), _ptr(t["wq"]), _ptr(t["scales"]), _ptr(t["zeros"]))
        assert L.gemv_q4_ws(*args, _ptr(y_ws), M, N, K, g, _ptr(ws), ws.numel(), stream) == q4.Q4_OK
        assert L.gemv_q4_static(*args, _ptr(y_st), M, N, K, g, stream) == q4.Q4_OK
        torch.cuda.synchronize()
        a, b = y_ws.cpu().numpy(), y_st.cpu().numpy()
        assert np.array_equal(a, b), f"call {i}: gemv_q4_static differs from gemv_q4_ws"
        rows = np.unique(np.r_[0:min(N, 64), max(0, N - 64):N])
        y_ref, bound = oracle.gemv_q4(d["x"], d["wq"], d["scales"], d["zeros"], g, rows=rows)
        err = np.abs(b[:, rows].astype(np.float64) - y_ref)
        assert (err <= oracle.gemv_tolerance(bound)).all(), f"call {i}: outside the GEMV bound"


def test_static_rejects_what_gemv_q4_rejects():
    L = q4.lib()
    A = ctypes.c_void_p(0x10000)
    assert L.gemv_q4_static(A, A, A, A, A, 1, 8, 100, 32, None) == q4.Q4_EINVAL
    assert L.gemv_q4_static(None, A, A, A, A, 8, 64, 14336, 128, None) == q4.Q4_ENULL
    assert L.gemv_q4_static(A, A, A, A, A, 8, 0, 14336, 128, None) == q4.Q4_OK
