"""The pins have teeth: plausible mistakes planted in the oracle are caught.

Each case monkeypatches one oracle function with a plausible error (a
dropped term, a wrong power, a wrong tie rule, a skipped step, an inverted
factor) and runs the pins that should catch it; at least one must fail.
Mistakes are planted in the oracle only, on the CPU.
"""

import numpy as np
import pytest

import tests.test_oracle_formats as TF
import tests.test_oracle_pins as TP
from oracle import dualquant as D
from oracle import formats as F


def _fails(*calls):
    for fn, kw in calls:
        try:
            fn(**kw)
        except (AssertionError, ValueError):
            return True
    return False


def test_round_half_up_is_caught(monkeypatch):
    monkeypatch.setattr(F, "round_int_grid",
                        lambda x, grid: np.clip(np.floor(np.asarray(x) + 0.5), *F.INT_GRIDS[grid]))
    assert _fails((TF.test_int_rounding_ties_to_even_and_clips, {}))


def test_e2m1_tie_to_odd_is_caught(monkeypatch):
    orig = F.round_e2m1

    def bad(x):
        x = np.asarray(x, dtype=np.float64)
        y = orig(x)
        ax = np.abs(x)
        up = np.isin(ax, [0.25, 1.25, 2.5, 5.0])       # take the odd neighbour
        nxt = {0.25: 0.5, 1.25: 1.5, 2.5: 3.0, 5.0: 6.0}
        for k, v in nxt.items():
            y = np.where(up & (ax == k), np.sign(x) * v, y)
        return y
    monkeypatch.setattr(F, "round_e2m1", bad)
    assert _fails((TF.test_e2m1_rounding_matches_brute_force_incl_every_midpoint, {}))


def test_projection_through_float32_is_caught(monkeypatch):
    orig = F.project
    monkeypatch.setattr(F, "project",
                        lambda x, fmt: orig(np.asarray(x, np.float64).astype(np.float32).astype(np.float64), fmt))
    assert _fails((TF.test_projection_double_rounding_trap, {}))


def test_wrong_power_of_b_in_row_update_is_caught(monkeypatch):
    def bad(W, Q, b, fmt):
        return D.__dict__["_orig_update_a"](W, Q, np.asarray(b) ** 2, fmt)
    monkeypatch.setitem(D.__dict__, "_orig_update_a", D.update_a)
    monkeypatch.setattr(D, "update_a", bad)
    assert _fails(*[(TP.test_row_update_is_brute_force_argmin, {"fmt": f, "seed": s})
                    for f in TP.FMTS for s in (0, 1, 2)])


def test_extra_factor_in_column_update_is_caught(monkeypatch):
    orig = D.update_b

    def bad(W, Q, a, fmt):
        return orig(W, Q, np.asarray(a) * 2.0, fmt)   # S = 2 a Q
    monkeypatch.setattr(D, "update_b", bad)
    assert _fails(*[(TP.test_column_update_is_brute_force_argmin, {"fmt": f, "seed": 0})
                    for f in TP.FMTS])


def test_missing_projection_is_caught(monkeypatch):
    def bad(W, Q, b, fmt):
        R = Q * b[None, :]
        num = D.block_sums(W * R, fmt.group)
        den = D.block_sums(R * R, fmt.group)
        return np.where(den > 0, num / np.where(den > 0, den, 1), 1.0)
    monkeypatch.setattr(D, "update_a", bad)
    assert _fails((TP.test_outputs_representable_positive_and_on_grid, {"fmt": D.INT4_G64}))


def test_zero_slice_scale_zero_is_caught(monkeypatch):
    orig = D.update_b

    def bad(W, Q, a, fmt):
        b = orig(W, Q, a, fmt)
        S = D.expand_blocks(a, fmt.group) * Q
        return np.where((S * S).sum(axis=0) > 0, b, 0.0)
    monkeypatch.setattr(D, "update_b", bad)
    assert _fails((TP.test_all_zero_code_slices_get_scale_one, {"fmt": D.INT4_G64}))


def test_wrong_qmax_in_init_is_caught(monkeypatch):
    monkeypatch.setitem(F.QMAX, "int4", 8.0)
    assert _fails((TP.test_t0_is_textbook_per_group_absmax_rtn, {"fmt": D.INT4_G64}))


def test_skipped_requant_between_updates_is_caught(monkeypatch):
    # Column update on the codes from before the row update: still a
    # fixed-code descent step, so only the exact re-run of the pages'
    # order catches it.
    def bad_solve(W, fmt, iters, a=None, b=None, history=False):
        W = np.asarray(W, dtype=np.float64)
        if a is None:
            a, b = D.init_rtn(W, fmt)
        Q = D.quantize(W, a, b, fmt)
        for _ in range(iters):
            a = D.update_a(W, Q, b, fmt)
            b = D.update_b(W, Q, a, fmt)
            Q = D.quantize(W, a, b, fmt)
        return D.Solution(a, b, Q)
    monkeypatch.setattr(D, "solve", bad_solve)
    assert _fails(*[(TP.test_float64_oracle_equals_exact_rational_arithmetic, {"fmt": f})
                    for f in TP.FMTS])


def test_inverse_column_fold_in_activations_is_caught(monkeypatch):
    orig = D.rescale_quantize_act
    monkeypatch.setattr(D, "rescale_quantize_act", lambda X, b, fmt: orig(X, 1.0 / np.asarray(b), fmt))
    assert _fails(*[(TP.test_activation_rescale_follows_the_factorization, {"fmt": f})
                    for f in TP.FMTS])


@pytest.mark.parametrize("axis_bug", ["rows"])
def test_column_sums_over_wrong_axis_is_caught(monkeypatch, axis_bug):
    # b from per-row sums broadcast back onto columns (a transposed operand)
    def bad(W, Q, a, fmt):
        S = D.expand_blocks(a, fmt.group) * Q
        num = (W * S).sum(axis=1)
        den = (S * S).sum(axis=1)
        r = np.resize(num / np.where(den > 0, den, 1), W.shape[1])
        return np.where(r > 0, F.project(np.where(r > 0, r, 1), fmt.b_fmt), 1.0)
    monkeypatch.setattr(D, "update_b", bad)
    assert _fails((TP.test_column_stripes_decouple, {"fmt": D.INT4_G64}),
                  (TP.test_column_update_is_brute_force_argmin, {"fmt": D.INT4_G64, "seed": 0}))


def _colnorm_pins():
    return [(TP.test_colnorm_init_rank_one_closed_form, {"fmt": f}) for f in TP.FMTS] + \
           [(TP.test_colnorm_init_equals_exact_rational_definition, {"fmt": f}) for f in TP.FMTS] + \
           [(TP.test_colnorm_init_zero_slices_and_column_equivariance, {"fmt": f}) for f in TP.FMTS]


def test_colnorm_max_instead_of_mean_is_caught(monkeypatch):
    def bad(W, fmt):
        W = np.asarray(W, dtype=np.float64)
        cm = np.abs(W).max(axis=0)
        b = np.where(cm > 0, F.project(np.where(cm > 0, cm, 1.0), fmt.b_fmt), 1.0)
        a, _ = D.init_rtn(W / b[None, :], fmt)
        return a, b
    monkeypatch.setattr(D, "init_colnorm", bad)
    assert _fails(*_colnorm_pins())


def test_colnorm_block_scales_without_column_division_are_caught(monkeypatch):
    orig = D.init_colnorm

    def bad(W, fmt):
        _, b = orig(W, fmt)
        a, _ = D.init_rtn(W, fmt)
        return a, b
    monkeypatch.setattr(D, "init_colnorm", bad)
    assert _fails(*_colnorm_pins())


def test_e4m3_element_ties_away_from_zero_is_caught(monkeypatch):
    def bad(x):
        x = np.asarray(x, dtype=np.float64)
        lv = F.e4m3_levels()
        ax = np.minimum(np.abs(x), lv[-1])
        hi = np.clip(np.searchsorted(lv, ax, side="left"), 1, len(lv) - 1)
        lo = hi - 1
        mag = np.where(lv[hi] - ax <= ax - lv[lo], lv[hi], lv[lo])    # ties go up
        return np.where(x < 0, -mag, mag) + 0.0
    monkeypatch.setattr(F, "round_e4m3", bad)
    assert _fails((TF.test_e4m3_elements_match_brute_force_and_torch, {}))


@pytest.mark.parametrize("bug", ["shifted_state", "changed_off_by_one"])
def test_iteration_stats_misaligned_rows_are_caught(monkeypatch, bug):
    # a row taken one sub-step early, or the changed counts shifted by one
    # iteration: the per-state recount must notice
    orig = D.iteration_stats

    def bad(W, fmt, iters, a=None, b=None):
        st = orig(W, fmt, iters, a, b)
        if bug == "shifted_state":
            sol = D.solve(W, fmt, iters, a, b, history=True)
            st[1:, 0] = sol.sse[3::4]        # after the column update, before requantizing
        else:
            st[1:-1, 2] = st[2:, 2]
        return st
    monkeypatch.setattr(D, "iteration_stats", bad)
    assert _fails((TP.test_iteration_stats_recount_every_state, {"fmt": D.INT4_G64}))
