"""Helpers for the GPU tests: run the HIP library through its C ABI and bring
results back as float64 numpy arrays decoded with the oracle's tables."""

from __future__ import annotations

import numpy as np
import torch

from calibration_free_bit_amd import dq
from oracle import dualquant as D
from oracle import formats as F

GRID_NAME = {dq.GRID_INT4: "int4", dq.GRID_E2M1: "e2m1", dq.GRID_INT8: "int8", dq.GRID_E4M3: "e4m3"}
AFMT_NAME = {dq.SCALE_FP16: "fp16", dq.SCALE_E8M0: "e8m0", dq.SCALE_E4M3: "e4m3"}

#: Every (grid, G, block-scale) combination the library builds, by name.
ALL_FORMATS = {f"{GRID_NAME[g]}_g{G}_{AFMT_NAME[a]}": dq.Format(g, G, a)
               for g in (dq.GRID_INT4, dq.GRID_E2M1, dq.GRID_INT8, dq.GRID_E4M3) for G in (16, 32, 64)
               for a in (dq.SCALE_FP16, dq.SCALE_E8M0, dq.SCALE_E4M3)}


def oracle_fmt(fmt: dq.Format) -> D.Format:
    return D.Format(GRID_NAME[fmt.grid], fmt.group, AFMT_NAME[fmt.a_fmt], "fp16")


def to_device(data: np.ndarray, ldw: int | None = None) -> torch.Tensor:
    """uint16 bf16 bits -> int16 device tensor; float32 -> float32 device
    tensor. With ldw > cols the rows are padded (pad filled with garbage)."""
    M, N = data.shape
    if ldw is not None and ldw != N:
        pad = np.full((M, ldw), 0x7F7F if data.dtype == np.uint16 else 3.0e38, dtype=data.dtype)
        pad[:, :N] = data
        data = pad
    host = torch.from_numpy(data.view(np.int16) if data.dtype == np.uint16 else data)
    t = host.cuda()
    return t[:, :N] if ldw is not None and ldw != N else t


def decode_a(a_t: torch.Tensor, fmt: dq.Format) -> np.ndarray:
    raw = a_t.cpu().numpy()
    raw = raw.view(np.uint16) if fmt.a_fmt == dq.SCALE_FP16 else raw.view(np.uint8)
    return F.decode_scale(raw, AFMT_NAME[fmt.a_fmt])


def decode_b(b_t: torch.Tensor) -> np.ndarray:
    return F.decode_scale(b_t.cpu().numpy().view(np.uint16), "fp16")


class DeviceRun:
    """One matrix on the GPU: init, iterate, pack through the C ABI."""

    def __init__(self, data: np.ndarray, fmt: dq.Format, ldw: int | None = None):
        self.fmt = fmt
        self.W = to_device(data, ldw)
        self.s = dq.Solver(self.W, fmt)

    def run(self, iters: int, init: bool = True):
        if init:
            self.s.init()
        self.s.iterate(iters)
        self.s.pack()
        torch.cuda.synchronize()
        return self

    def solve(self, iters: int):
        """The same work as one dq_solve call (the benchmark's step)."""
        self.s.solve(iters)
        torch.cuda.synchronize()
        return self

    @property
    def a(self):
        return decode_a(self.s.a, self.fmt)

    @property
    def b(self):
        return decode_b(self.s.b)

    @property
    def Q(self):
        return D.unpack_codes(self.s.packed.cpu().numpy(), oracle_fmt(self.fmt))

    @property
    def packed(self):
        return self.s.packed.cpu().numpy()


def as_f64(data: np.ndarray) -> np.ndarray:
    from calibration_free_bit_amd import synth
    return synth.bf16_to_f64(data) if data.dtype == np.uint16 else data.astype(np.float64)


def compare(W64, gpu_a, gpu_b, gpu_Q, sol: D.Solution, ofmt: D.Format, what=""):
    """The parity bar: scales within 1e-5 relative (reported as exact
    mismatch counts too), codes identical except at exact rounding ties of
    the oracle, reconstruction SSE within 1e-5 relative."""
    ra = np.abs(gpu_a - sol.a) / sol.a
    rb = np.abs(gpu_b - sol.b) / sol.b
    assert ra.max() <= 1e-5, f"{what}: a max rel err {ra.max()} ({(gpu_a != sol.a).sum()} differ)"
    assert rb.max() <= 1e-5, f"{what}: b max rel err {rb.max()} ({(gpu_b != sol.b).sum()} differ)"
    diff = gpu_Q != sol.Q
    if diff.any():
        ties = D.code_ties(W64, sol.a, sol.b, ofmt)
        assert np.all(ties[diff]), f"{what}: {int((diff & ~ties).sum())} non-tie code mismatches"
        assert diff.mean() <= 1e-4, f"{what}: {diff.mean()} of codes differ"
    s_gpu = D.sse(W64, gpu_a, gpu_Q, gpu_b, ofmt)
    s_ref = D.sse(W64, sol.a, sol.Q, sol.b, ofmt)
    assert abs(s_gpu - s_ref) <= 1e-5 * max(s_ref, 1e-300), f"{what}: SSE {s_gpu} vs {s_ref}"
    return {"a_diff": int((gpu_a != sol.a).sum()), "b_diff": int((gpu_b != sol.b).sum()),
            "q_diff": int(diff.sum())}
