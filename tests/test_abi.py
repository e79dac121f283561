"""The C-ABI library loads and exports what include/dq.h declares; host-side
argument validation returns status codes without launching anything.

No compute call is made here (no GPU needed): every call below fails
validation on the host before any HIP API is touched.
"""

import ctypes
import os
import re

import pytest

from calibration_free_bit_amd import dq, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "dq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dq_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    declared = _declared_functions()
    assert declared == sorted(dq.EXPORTS)
    L = dq.lib()
    for name in declared:
        assert hasattr(L, name), name


def test_library_has_gfx950_code_object():
    blob = open(dq.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def test_status_strings_and_version():
    assert dq.abi_version() == 1
    L = dq.lib()
    for s in (0, -1, -2, -3, -4, -5):
        assert L.dq_status_string(s)
    assert L.dq_status_string(-99) == b"unknown status"


def _p(**kw):
    base = dict(rows=64, cols=128, ldw=128, group=64, grid=dq.GRID_INT4, a_fmt=dq.SCALE_FP16,
                b_fmt=dq.SCALE_FP16, w_type=dq.W_BF16, reserved=0)
    base.update(kw)
    return dq.Problem(**base)


def test_stats_workspace_holds_one_state_of_codes():
    L = dq.lib()
    for grid, bits in ((dq.GRID_INT4, 4), (dq.GRID_E2M1, 4), (dq.GRID_INT8, 8), (dq.GRID_E4M3, 8)):
        p = _p(rows=300, cols=576, ldw=576, grid=grid)
        base = L.dq_workspace_bytes(ctypes.byref(p))
        st = L.dq_stats_workspace_bytes(ctypes.byref(p))
        assert st >= base + 300 * 576 * bits // 8
    assert L.dq_stats_workspace_bytes(ctypes.byref(_p(cols=100))) == 0
    assert L.dq_stats_workspace_bytes(None) == 0


def test_workspace_bytes_valid_and_invalid():
    L = dq.lib()
    nb = L.dq_workspace_bytes(ctypes.byref(_p()))
    assert nb > 0 and nb % 256 == 0
    assert L.dq_workspace_bytes(ctypes.byref(_p(cols=100))) == 0          # cols % G
    assert L.dq_workspace_bytes(ctypes.byref(_p(group=8))) == 0
    assert L.dq_workspace_bytes(ctypes.byref(_p(ldw=120))) == 0           # ldw < cols
    assert L.dq_workspace_bytes(None) == 0
    big = L.dq_workspace_bytes(ctypes.byref(_p(rows=14336, cols=4096, ldw=4096, group=32,
                                                a_fmt=dq.SCALE_E8M0)))
    assert 0 < big < 64 << 20


@pytest.mark.parametrize("kw,status", [
    (dict(cols=100), dq.ERR_SHAPE),
    (dict(rows=0), dq.ERR_SHAPE),
    (dict(ldw=132), dq.ERR_SHAPE),             # 132 * 2 bytes is not a multiple of 16
    (dict(ldw=1 << 31), dq.ERR_SHAPE),         # geometry is passed as 32-bit arguments
    (dict(rows=1 << 31, ldw=128), dq.ERR_SHAPE),
    (dict(group=128), dq.ERR_UNSUPPORTED),
    (dict(grid=7), dq.ERR_UNSUPPORTED),
    (dict(a_fmt=9), dq.ERR_UNSUPPORTED),
    (dict(b_fmt=dq.SCALE_E8M0), dq.ERR_UNSUPPORTED),
    (dict(w_type=5), dq.ERR_UNSUPPORTED),
])
def test_bad_problems_are_rejected_on_host(kw, status):
    L = dq.lib()
    p = _p(**kw)
    fake = ctypes.c_void_p(256)      # never dereferenced: validation fails first
    assert L.dq_init_rtn(ctypes.byref(p), fake, fake, fake, None) == status
    assert L.dq_pack_codes(ctypes.byref(p), fake, fake, fake, fake, None) == status
    assert L.dq_bcd_iterate(ctypes.byref(p), fake, fake, fake, 1, fake, 1 << 20, None, None) == status


def test_null_and_misaligned_pointers_are_rejected():
    L = dq.lib()
    p = _p()
    ok = ctypes.c_void_p(256)
    assert L.dq_init_rtn(ctypes.byref(p), None, ok, ok, None) == dq.ERR_INVALID_ARG
    assert L.dq_init_rtn(ctypes.byref(p), ctypes.c_void_p(258), ok, ok, None) == dq.ERR_INVALID_ARG
    assert L.dq_init_rtn(None, ok, ok, ok, None) == dq.ERR_INVALID_ARG
    assert L.dq_bcd_iterate(ctypes.byref(p), ok, ok, ok, -1, ok, 1 << 20, None, None) == dq.ERR_INVALID_ARG
    assert L.dq_pack_codes(ctypes.byref(p), ok, ok, ok, ctypes.c_void_p(259), None) == dq.ERR_INVALID_ARG
    assert L.dq_pack_codes(ctypes.byref(p), ok, ok, ctypes.c_void_p(258), ok, None) == dq.ERR_INVALID_ARG


def test_init_colnorm_checks_arguments_before_launch():
    L = dq.lib()
    p = _p()
    ok = ctypes.c_void_p(256)
    need = L.dq_workspace_bytes(ctypes.byref(p))
    assert need > 0
    assert L.dq_init_colnorm(ctypes.byref(p), None, ok, ok, ok, need, None) == dq.ERR_INVALID_ARG
    assert L.dq_init_colnorm(ctypes.byref(p), ctypes.c_void_p(264), ok, ok, ok, need, None) == dq.ERR_INVALID_ARG
    assert L.dq_init_colnorm(ctypes.byref(p), ok, ok, ok, None, need, None) == dq.ERR_WORKSPACE
    assert L.dq_init_colnorm(ctypes.byref(p), ok, ok, ok, ok, need - 1, None) == dq.ERR_WORKSPACE
    assert L.dq_init_colnorm(ctypes.byref(p), ok, ok, ok, ctypes.c_void_p(128), need, None) == dq.ERR_WORKSPACE


def test_quant_report_checks_arguments_before_launch():
    L = dq.lib()
    p = _p()
    ok = ctypes.c_void_p(256)
    need = L.dq_workspace_bytes(ctypes.byref(p))
    assert L.dq_quant_report(ctypes.byref(p), ok, ok, ok, None, None, None, ok, need, None) == dq.ERR_INVALID_ARG
    assert L.dq_quant_report(ctypes.byref(p), ok, ok, ctypes.c_void_p(258), None, None, ok, ok, need,
                             None) == dq.ERR_INVALID_ARG
    assert L.dq_quant_report(ctypes.byref(p), ok, ok, ok, ctypes.c_void_p(260), None, ok, ok, need,
                             None) == dq.ERR_INVALID_ARG
    assert L.dq_quant_report(ctypes.byref(p), ok, ok, ok, None, None, ok, None, need, None) == dq.ERR_WORKSPACE
    assert L.dq_quant_report(ctypes.byref(p), ok, ok, ok, None, None, ok, ok, need - 8, None) == dq.ERR_WORKSPACE


def test_iterate_checks_workspace_and_stats_before_launch():
    L = dq.lib()
    p = _p()
    ok = ctypes.c_void_p(256)
    need = L.dq_workspace_bytes(ctypes.byref(p))
    assert L.dq_bcd_iterate(ctypes.byref(p), ok, ok, ok, 1, ok, need - 1, None, None) == dq.ERR_WORKSPACE
    assert L.dq_bcd_iterate(ctypes.byref(p), ok, ok, ok, 1, None, need, None, None) == dq.ERR_WORKSPACE
    assert L.dq_bcd_iterate(ctypes.byref(p), ok, ok, ok, 1, ctypes.c_void_p(264), need, None,
                            None) == dq.ERR_WORKSPACE            # not 256-byte aligned
    # statistics need the larger workspace and an 8-byte aligned array
    need_st = L.dq_stats_workspace_bytes(ctypes.byref(p))
    assert need_st >= need and need_st % 256 == 0
    assert L.dq_bcd_iterate(ctypes.byref(p), ok, ok, ok, 1, ok, need, ok, None) == dq.ERR_WORKSPACE
    assert L.dq_bcd_iterate(ctypes.byref(p), ok, ok, ok, 1, ok, need_st - 1, ok, None) == dq.ERR_WORKSPACE
    assert L.dq_bcd_iterate(ctypes.byref(p), ok, ok, ok, 1, ok, need_st, ctypes.c_void_p(260),
                            None) == dq.ERR_INVALID_ARG
    # zero iterations is a no-op that touches nothing; with statistics it
    # writes row 0, so it needs the workspace
    assert L.dq_bcd_iterate(ctypes.byref(p), ok, ok, ok, 0, None, 0, None, None) == dq.OK
    assert L.dq_bcd_iterate(ctypes.byref(p), ok, ok, ok, 0, None, 0, ok, None) == dq.ERR_WORKSPACE


def test_noalloc_iterate_checks_arguments_before_launch():
    L = dq.lib()
    p = _p()
    ok = ctypes.c_void_p(256)
    f = L.dq_bcd_iterate_noalloc
    assert f(ctypes.byref(p), None, ok, ok, 1, None) == dq.ERR_INVALID_ARG
    assert f(ctypes.byref(p), ok, None, ok, 1, None) == dq.ERR_INVALID_ARG
    assert f(ctypes.byref(p), ctypes.c_void_p(264), ok, ok, 1, None) == dq.ERR_INVALID_ARG
    assert f(ctypes.byref(p), ok, ok, ok, -1, None) == dq.ERR_INVALID_ARG
    assert f(ctypes.byref(_p(cols=100)), ok, ok, ok, 1, None) == dq.ERR_SHAPE
    # partial sums larger than the library's fixed scratch (16 MiB)
    big = dq.problem(64, 1 << 20, dq.FORMATS["int4_g64"], dq.W_BF16)
    assert L.dq_workspace_bytes(ctypes.byref(big)) > 16 << 20
    assert f(ctypes.byref(big), ok, ok, ok, 1, None) == dq.ERR_WORKSPACE
    # zero iterations touch nothing
    assert f(ctypes.byref(p), ok, ok, ok, 0, None) == dq.OK


def test_solve_checks_arguments_before_launch():
    L = dq.lib()
    p = _p()
    ok = ctypes.c_void_p(256)
    need = L.dq_workspace_bytes(ctypes.byref(p))
    assert L.dq_solve(ctypes.byref(p), ok, ok, ok, 3, None, ok, need, None) == dq.ERR_INVALID_ARG
    assert L.dq_solve(ctypes.byref(p), ok, ok, ok, -1, ok, ok, need, None) == dq.ERR_INVALID_ARG
    assert L.dq_solve(ctypes.byref(p), ok, ok, ctypes.c_void_p(258), 3, ok, ok, need, None) == dq.ERR_INVALID_ARG
    assert L.dq_solve(ctypes.byref(p), ok, ok, ok, 3, ctypes.c_void_p(260), ok, need, None) == dq.ERR_INVALID_ARG
    assert L.dq_solve(ctypes.byref(p), ok, ok, ok, 3, ok, ok, need - 1, None) == dq.ERR_WORKSPACE
    assert L.dq_solve(ctypes.byref(_p(cols=100)), ok, ok, ok, 3, ok, ok, need, None) == dq.ERR_SHAPE


def test_activation_call_validation():
    L = dq.lib()
    p = _p()
    ok = ctypes.c_void_p(256)
    assert L.dq_rescale_quantize_act(ctypes.byref(_p(w_type=dq.W_F32)), ok, 4, 128, ok, ok, ok,
                                     None) == dq.ERR_UNSUPPORTED
    assert L.dq_rescale_quantize_act(ctypes.byref(p), ok, -1, 128, ok, ok, ok, None) == dq.ERR_SHAPE
    assert L.dq_rescale_quantize_act(ctypes.byref(p), ok, 4, 64, ok, ok, ok, None) == dq.ERR_SHAPE
    assert L.dq_rescale_quantize_act(ctypes.byref(p), ok, 0, 128, ok, ok, ok, None) == dq.OK
    assert L.dq_rescale_quantize_act(ctypes.byref(p), None, 4, 128, ok, ok, ok, None) == dq.ERR_INVALID_ARG


def test_binding_fails_loudly_without_the_library(monkeypatch):
    monkeypatch.setattr(dq, "_lib", None)
    monkeypatch.setattr(dq, "LIB_PATH", "/nonexistent/libdq.so")
    with pytest.raises(RuntimeError, match="HIP library not found"):
        dq.lib()


def test_assign_streams_is_balanced_and_deterministic():
    # host-side scheduling of the set workload: greedy longest-first
    sizes = [sp.rows * sp.cols for _, _, _, sp, _ in synth.llama_layer_specs()]
    w = dq.assign_streams(sizes, 4)
    assert w == dq.assign_streams(sizes, 4)
    load = [sum(s for s, j in zip(sizes, w) if j == k) for k in range(4)]
    assert max(load) - min(load) <= max(sizes)
    assert dq.assign_streams([5, 3, 3, 1], 2) == [0, 1, 1, 0]
