"""dq_bcd_iterate_noalloc (no workspace argument, nothing allocated) against
dq_bcd_iterate on the same inputs: a and b must come out bit for bit the
same. Two calls in a row, the second on a smaller problem, so that the
library's fixed scratch still holds the first call's partial sums when the
second runs."""

import numpy as np
import pytest
import torch

from calibration_free_bit_amd import dq, synth
from tests.gpu_util import to_device

pytestmark = pytest.mark.gpu


def _matrix(M, N, seed):
    spec = synth.MatrixSpec(M, N, "normal", 0.02, 0.01, (20.0, 20.0), "bf16")
    return synth.make_matrix(spec, seed).data


def _pair(name, M, N, iters, seed):
    """Both entry points from the same absmax start; returns the two Solvers."""
    print(f"[case] noalloc {name} {M}x{N} T={iters} seed {seed}", flush=True)
    fmt = dq.FORMATS[name]
    W = to_device(_matrix(M, N, seed))
    ref = dq.Solver(W, fmt)
    ref.init()
    ref.iterate(iters)
    got = dq.Solver(W, fmt)
    got.init()
    dq.bcd_iterate_noalloc(got.p, W, got.a, got.b, iters)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_equals_iterate_on_two_calls_second_smaller():
    for name, M, N, iters, seed in (("nvfp4_g16", 4096, 14336, 4, 11),
                                    ("int4_g64", 300, 576, 3, 12)):
        ref, got = _pair(name, M, N, iters, seed)
        assert torch.equal(ref.a, got.a), (name, M, N)
        assert torch.equal(ref.b, got.b), (name, M, N)


def test_noalloc_composes_and_rejects_oversized_problems():
    # iterate(2) then iterate(3) through the fixed scratch equals iterate(5)
    fmt = dq.FORMATS["mxint4_g32"]
    W = to_device(_matrix(1024, 4096, 13))
    ref = dq.Solver(W, fmt)
    ref.init()
    ref.iterate(5)
    got = dq.Solver(W, fmt)
    got.init()
    dq.bcd_iterate_noalloc(got.p, W, got.a, got.b, 2)
    dq.bcd_iterate_noalloc(got.p, W, got.a, got.b, 3)
    torch.cuda.synchronize()
    assert torch.equal(ref.a, got.a) and torch.equal(ref.b, got.b)
    # a problem whose partial sums exceed the fixed scratch is refused
    # before anything is launched, and leaves a and b untouched
    big = dq.problem(64, 1 << 20, dq.FORMATS["int4_g64"], dq.W_BF16)
    assert dq.workspace_bytes(big) > 16 << 20
    a0, b0 = got.a.clone(), got.b.clone()
    with pytest.raises(dq.DQError) as e:
        dq.bcd_iterate_noalloc(big, W, got.a, got.b, 1)
    assert e.value.status == dq.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(a0, got.a) and torch.equal(b0, got.b)
