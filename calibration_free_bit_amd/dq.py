"""ctypes binding of libdq.so: the C ABI of include/dq.h, same names.

Argument marshalling only: every step of the solver runs in the HIP
library. PyTorch supplies device memory and the stream; tensors are passed
by data pointer. The library is loaded on first use from the in-tree build
(``calibration_free_bit_amd/_lib/libdq.so``); if it is missing the call
raises -- there is no fallback of any kind.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("DQ_LIB_PATH", os.path.join(_HERE, "_lib", "libdq.so"))

# enums of dq.h
OK, ERR_INVALID_ARG, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4, -5
GRID_INT4, GRID_E2M1, GRID_INT8, GRID_E4M3 = 0, 1, 2, 3
SCALE_FP16, SCALE_E8M0, SCALE_E4M3 = 0, 1, 2
W_F32, W_BF16 = 0, 1

EXPORTS = ("dq_workspace_bytes", "dq_stats_workspace_bytes", "dq_init_rtn", "dq_init_colnorm",
           "dq_bcd_iterate", "dq_bcd_iterate_noalloc", "dq_solve", "dq_pack_codes", "dq_quant_report", "dq_rescale_quantize_act",
           "dq_status_string", "dq_abi_version")


class Problem(ctypes.Structure):
    """dq_problem of dq.h."""
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("ldw", ctypes.c_int64),
                ("group", ctypes.c_int32), ("grid", ctypes.c_int32), ("a_fmt", ctypes.c_int32),
                ("b_fmt", ctypes.c_int32), ("w_type", ctypes.c_int32), ("reserved", ctypes.c_int32)]


@dataclass(frozen=True)
class Format:
    """A quantization format: element grid, block size, block-scale set."""
    grid: int
    group: int
    a_fmt: int

    @property
    def a_dtype(self):
        return torch.int16 if self.a_fmt == SCALE_FP16 else torch.uint8

    @property
    def code_bits(self) -> int:
        return 8 if self.grid in (GRID_INT8, GRID_E4M3) else 4


#: Formats of the DualQuant summary §3 and §G.2 (column scales are fp16 for all).
FORMATS = {
    "int4_g64": Format(GRID_INT4, 64, SCALE_FP16),
    "mxint4_g32": Format(GRID_INT4, 32, SCALE_E8M0),
    "nvfp4_g16": Format(GRID_E2M1, 16, SCALE_E4M3),
    "mxfp4_g32": Format(GRID_E2M1, 32, SCALE_E8M0),
    "mxint8_g32": Format(GRID_INT8, 32, SCALE_E8M0),
    "mxfp8_g32": Format(GRID_E4M3, 32, SCALE_E8M0),
}


class DQError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdq.so (once). Raises if the HIP library was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library not found at {LIB_PATH}; build it with "
                "`python -m calibration_free_bit_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Problem)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.dq_workspace_bytes.argtypes, L.dq_workspace_bytes.restype = [P], sz
        L.dq_stats_workspace_bytes.argtypes, L.dq_stats_workspace_bytes.restype = [P], sz
        L.dq_init_rtn.argtypes, L.dq_init_rtn.restype = [P, vp, vp, vp, vp], ctypes.c_int
        L.dq_init_colnorm.argtypes = [P, vp, vp, vp, vp, sz, vp]
        L.dq_init_colnorm.restype = ctypes.c_int
        L.dq_bcd_iterate.argtypes = [P, vp, vp, vp, i32, vp, sz, vp, vp]
        L.dq_bcd_iterate.restype = ctypes.c_int
        L.dq_bcd_iterate_noalloc.argtypes = [P, vp, vp, vp, i32, vp]
        L.dq_bcd_iterate_noalloc.restype = ctypes.c_int
        L.dq_solve.argtypes, L.dq_solve.restype = [P, vp, vp, vp, i32, vp, vp, sz, vp], ctypes.c_int
        L.dq_pack_codes.argtypes, L.dq_pack_codes.restype = [P, vp, vp, vp, vp, vp], ctypes.c_int
        L.dq_quant_report.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.dq_quant_report.restype = ctypes.c_int
        L.dq_rescale_quantize_act.argtypes = [P, vp, i64, i64, vp, vp, vp, vp]
        L.dq_rescale_quantize_act.restype = ctypes.c_int
        L.dq_status_string.argtypes, L.dq_status_string.restype = [ctypes.c_int], ctypes.c_char_p
        L.dq_abi_version.argtypes, L.dq_abi_version.restype = [], ctypes.c_int
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise DQError(fn, status, lib().dq_status_string(status).decode())


def problem(rows: int, cols: int, fmt: Format, w_type: int, ldw: int | None = None) -> Problem:
    return Problem(rows, cols, cols if ldw is None else ldw, fmt.group, fmt.grid, fmt.a_fmt,
                   SCALE_FP16, w_type, 0)


def problem_for(W: torch.Tensor, fmt: Format) -> Problem:
    """dq_problem describing a 2-D weight tensor (float32, or bf16 given as
    torch.bfloat16 or as its uint16 bit patterns in an int16 tensor) whose
    rows are contiguous (any row pitch)."""
    if W.dtype == torch.float32:
        w_type = W_F32
    elif W.dtype in (torch.bfloat16, torch.int16):
        w_type = W_BF16
    else:
        raise TypeError(f"W must be float32, bfloat16 or int16 (bf16 bits), not {W.dtype}")
    if W.dim() != 2 or (W.shape[1] > 1 and W.stride(1) != 1):
        raise ValueError("W must be a 2-D tensor with contiguous rows (stride(1) == 1)")
    return problem(W.shape[0], W.shape[1], fmt, w_type, W.stride(0))


def workspace_bytes(p: Problem) -> int:
    return int(lib().dq_workspace_bytes(ctypes.byref(p)))


def stats_workspace_bytes(p: Problem) -> int:
    return int(lib().dq_stats_workspace_bytes(ctypes.byref(p)))


def init_rtn(p: Problem, W, a, b, stream=None) -> None:
    _check("dq_init_rtn", lib().dq_init_rtn(ctypes.byref(p), _ptr(W), _ptr(a), _ptr(b), _stream(stream)))


def init_colnorm(p: Problem, W, a, b, workspace, workspace_nbytes: int | None = None,
                 stream=None) -> None:
    nbytes = workspace.numel() * workspace.element_size() if workspace_nbytes is None else workspace_nbytes
    _check("dq_init_colnorm", lib().dq_init_colnorm(
        ctypes.byref(p), _ptr(W), _ptr(a), _ptr(b), _ptr(workspace), int(nbytes), _stream(stream)))


def bcd_iterate(p: Problem, W, a, b, n_iters: int, workspace, workspace_nbytes: int | None = None,
                stats=None, stream=None) -> None:
    nbytes = workspace.numel() * workspace.element_size() if workspace_nbytes is None else workspace_nbytes
    _check("dq_bcd_iterate", lib().dq_bcd_iterate(
        ctypes.byref(p), _ptr(W), _ptr(a), _ptr(b), int(n_iters), _ptr(workspace), int(nbytes),
        _ptr(stats), _stream(stream)))


def bcd_iterate_noalloc(p: Problem, W, a, b, n_iters: int, stream=None) -> None:
    _check("dq_bcd_iterate_noalloc", lib().dq_bcd_iterate_noalloc(
        ctypes.byref(p), _ptr(W), _ptr(a), _ptr(b), int(n_iters), _stream(stream)))


def solve(p: Problem, W, a, b, n_iters: int, packed, workspace, workspace_nbytes: int | None = None,
          stream=None) -> None:
    nbytes = workspace.numel() * workspace.element_size() if workspace_nbytes is None else workspace_nbytes
    _check("dq_solve", lib().dq_solve(
        ctypes.byref(p), _ptr(W), _ptr(a), _ptr(b), int(n_iters), _ptr(packed), _ptr(workspace), int(nbytes),
        _stream(stream)))


def pack_codes(p: Problem, W, a, b, packed, stream=None) -> None:
    _check("dq_pack_codes", lib().dq_pack_codes(
        ctypes.byref(p), _ptr(W), _ptr(a), _ptr(b), _ptr(packed), _stream(stream)))


def quant_report(p: Problem, W, a, b, prev_packed, packed, report, workspace,
                 workspace_nbytes: int | None = None, stream=None) -> None:
    nbytes = workspace.numel() * workspace.element_size() if workspace_nbytes is None else workspace_nbytes
    _check("dq_quant_report", lib().dq_quant_report(
        ctypes.byref(p), _ptr(W), _ptr(a), _ptr(b), _ptr(prev_packed), _ptr(packed), _ptr(report),
        _ptr(workspace), int(nbytes), _stream(stream)))


def rescale_quantize_act(p: Problem, X, tokens: int, ldx: int, b, xq, x_scales, stream=None) -> None:
    _check("dq_rescale_quantize_act", lib().dq_rescale_quantize_act(
        ctypes.byref(p), _ptr(X), int(tokens), int(ldx), _ptr(b), _ptr(xq), _ptr(x_scales),
        _stream(stream)))


def abi_version() -> int:
    return int(lib().dq_abi_version())


# ------------------------------------------------------------------ helpers

class Solver:
    """Device buffers for one matrix: a, b, workspace, packed codes.

    ``solve(T)`` = dq_init_rtn, dq_bcd_iterate(T), dq_pack_codes on the
    current stream. Buffers are allocated once, at construction.
    """

    def __init__(self, W: torch.Tensor, fmt: Format):
        if W.dim() != 2 or not W.is_cuda:
            raise ValueError("W must be a 2-D device tensor")
        self.W, self.fmt = W, fmt
        self.p = problem_for(W, fmt)
        M, N = W.shape
        dev = W.device
        self.a = torch.empty((M, N // fmt.group), dtype=fmt.a_dtype, device=dev)
        self.b = torch.empty((N,), dtype=torch.int16, device=dev)
        nb = workspace_bytes(self.p)
        if nb == 0:
            raise DQError("dq_workspace_bytes", ERR_SHAPE, "invalid problem")
        self.ws = torch.empty((nb,), dtype=torch.uint8, device=dev)
        self.packed = torch.empty((M, N * fmt.code_bits // 8), dtype=torch.uint8, device=dev)

    def init(self, stream=None):
        init_rtn(self.p, self.W, self.a, self.b, stream)

    def init_colnorm(self, stream=None):
        init_colnorm(self.p, self.W, self.a, self.b, self.ws, stream=stream)

    def iterate(self, n: int, stream=None, stats: bool = False):
        """n BCD iterations; with ``stats`` returns the device tensor
        [n + 1, 3] of dq_bcd_iterate's per-iteration statistics (the larger
        workspace they need is allocated on first use)."""
        if not stats:
            bcd_iterate(self.p, self.W, self.a, self.b, n, self.ws, stream=stream)
            return None
        need = stats_workspace_bytes(self.p)
        # allocate (and clear) on the stream the call runs on, so that the
        # kernels are ordered after the fill
        if isinstance(stream, int):
            raise ValueError("iterate(stats=True) needs a torch stream (or None)")
        with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
            if self.ws.numel() < need:
                self.ws = torch.empty((need,), dtype=torch.uint8, device=self.W.device)
            out = torch.zeros((n + 1, 3), dtype=torch.float64, device=self.W.device)
        bcd_iterate(self.p, self.W, self.a, self.b, n, self.ws, stats=out, stream=stream)
        return out

    def pack(self, stream=None):
        pack_codes(self.p, self.W, self.a, self.b, self.packed, stream)

    def report(self, prev_packed=None, stream=None) -> torch.Tensor:
        """Codes of the current state into ``packed`` plus a device tensor
        [sum (W - a Q b)^2, sum W^2, codes differing from prev_packed]."""
        out = torch.empty(3, dtype=torch.float64, device=self.W.device)
        quant_report(self.p, self.W, self.a, self.b, prev_packed, self.packed, out, self.ws, stream=stream)
        return out

    def solve(self, iters: int = 15, stream=None):
        """init, ``iters`` iterations (15 by default, the count the DualQuant
        summary §5.3 uses), pack -- one dq_solve call, whose first pass
        forms the initialization itself."""
        solve(self.p, self.W, self.a, self.b, iters, self.packed, self.ws, stream=stream)

    def solve_until_stable(self, max_iters: int = 15, stream=None) -> int:
        """init, then iterations one at a time until one changes no code
        (the convergence criterion the summary §5.3 and App. B follow) or
        ``max_iters`` have run; then pack. Returns the iterations run. The
        state after k iterations is the one iterate(k) gives; each step
        reads its changed-code count back to the host."""
        if isinstance(stream, int):
            raise ValueError("solve_until_stable needs a torch stream (or None)")
        waiter = stream if stream is not None else torch.cuda.current_stream()
        self.init(stream)
        done = 0
        while done < max_iters:
            st = self.iterate(1, stream, stats=True)
            done += 1
            waiter.synchronize()
            if int(st[1, 2].item()) == 0:
                break
        self.pack(stream)
        return done


def assign_streams(sizes, n_streams: int):
    """Greedy longest-first assignment of matrices (by element count) to
    streams: returns the stream index of every matrix. Deterministic."""
    load = [0] * n_streams
    out = [0] * len(sizes)
    for k in sorted(range(len(sizes)), key=lambda k: (-sizes[k], k)):
        j = min(range(n_streams), key=lambda j: (load[j], j))
        out[k] = j
        load[j] += sizes[k]
    return out


def solve_on_streams(solvers, iters: int, streams) -> None:
    """solve(iters) for every solver, the matrices spread over ``streams``
    (forked from and joined back into the current stream), so that passes of
    different matrices overlap on the device. Each stream takes its matrices
    largest first, so that matrices of like size run side by side (for the
    Llama-3.1-8B set on two streams, 86.3 ms per step against 87.7 ms in
    layer order)."""
    cur = torch.cuda.current_stream()
    sizes = [s.W.shape[0] * s.W.shape[1] for s in solvers]
    where = assign_streams(sizes, len(streams))
    for st in streams:
        st.wait_stream(cur)
    for k in sorted(range(len(solvers)), key=lambda k: (-sizes[k], k)):
        solvers[k].solve(iters, streams[where[k]])
    for st in streams:
        cur.wait_stream(st)
