"""Pins of the oracle's number formats against definitions other than itself.

Element grids: [DQ summary] §3 (round-and-clip for integers, nearest level
for floating-point grids); scale sets: [DQ summary] §3 (fp16 / E8M0 /
UE4M3); projection: [DQ repro] "Core equations" (closest storable inverse
scale). Independent references used here: numpy's float16 cast,
torch's float8_e4m3fn dtype, the E2M1 bit layout, and brute force over the
whole legal set.
"""

import numpy as np
import pytest
import torch

from oracle import formats as F

RNG = np.random.default_rng(1234)


# ------------------------------------------------------------ element grids

def test_int4_grid_is_signed_4bit():
    # [SQuant tutorial] Ch. 2: 4-bit signed weights span [-8, 7].
    assert list(F.grid_codes("int4")) == list(range(-8, 8))


def test_e2m1_levels_match_bit_layout():
    # E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is
    # subnormal (value m/2). Decode all 16 codes from the bit definition.
    vals = set()
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = (m / 2.0) if e == 0 else 2.0 ** (e - 1) * (1 + m / 2.0)
        vals.add(-mag if s else mag)
    assert sorted(vals) == list(F.grid_codes("e2m1"))
    assert list(F.E2M1_LEVELS) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_int_rounding_ties_to_even_and_clips():
    x = np.array([-9.0, -8.5, -7.5, -2.5, -0.5, 0.5, 1.5, 2.5, 6.5, 7.49, 7.5, 9.0])
    got = F.round_int_grid(x, "int4")
    assert list(got) == [-8, -8, -8, -2, 0, 0, 2, 2, 6, 7, 7, 7]


def _e2m1_brute(x):
    """Nearest of all 15 E2M1 values by brute force; at a tie, the even code."""
    vals, codes = [], []
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = (m / 2.0) if e == 0 else 2.0 ** (e - 1) * (1 + m / 2.0)
        if code == 8:       # -0 duplicates +0
            continue
        vals.append(-mag if s else mag)
        codes.append(code & 7)
    vals, codes = np.array(vals), np.array(codes)
    out = []
    for xi in x:
        d = np.abs(vals - xi)
        best = np.flatnonzero(d == d.min())
        pick = [i for i in best if codes[i] % 2 == 0] or list(best)
        out.append(vals[pick[0]])
    return np.array(out)


def test_e2m1_rounding_matches_brute_force_incl_every_midpoint():
    g = F.grid_codes("e2m1")
    mids = (g[1:] + g[:-1]) / 2
    x = np.concatenate([mids, RNG.uniform(-8, 8, 3000), [7.0, -7.0, 6.0, 100.0, -0.0]])
    np.testing.assert_array_equal(F.round_e2m1(x), _e2m1_brute(x))
    # the tie rule on the positive midpoints: 0.25->0, 0.75->1, 1.25->1,
    # 1.75->2, 2.5->2, 3.5->4, 5->4
    pos = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert list(F.round_e2m1(pos)) == [0, 1, 1, 2, 2, 4, 4]
    assert list(F.round_e2m1(-pos)) == [0, -1, -1, -2, -2, -4, -4]
    assert not np.signbit(F.round_e2m1(np.array([-0.1])))[0]


def test_huge_magnitudes_saturate_on_every_grid():
    """Above the largest level the nearest level is the largest one, for any
    magnitude ([DQ summary] §3 formats; reading: saturation). Far above it
    float64 cannot tell the levels' distances apart, so the rounding must
    not rely on them there."""
    big = np.array([500.0 * 2.0 ** k for k in (0, 20, 60, 200, 1000)] + [np.inf])
    x = np.concatenate([big, -big])
    top = {"e2m1": 6.0, "e4m3": 448.0}
    for grid in ("e2m1", "e4m3"):
        want = np.where(x < 0, -top[grid], top[grid])
        np.testing.assert_array_equal(F.round_to_grid(x, grid), want)
    for grid in ("int4", "int8"):
        lo, hi = F.INT_GRIDS[grid]
        np.testing.assert_array_equal(F.round_to_grid(x, grid), np.where(x < 0, lo, hi))


def test_tie_mask_flags_exact_midpoints_only():
    x = np.array([0.5, 0.5000001, 2.5, -7.5, 7.5, -8.5, 3.0])
    assert list(F.tie_mask(x, "int4")) == [True, False, True, True, False, False, False]
    assert list(F.tie_mask(np.array([5.0, 2.5, 2.0]), "e2m1")) == [True, True, False]


def test_nibble_round_trip():
    for grid in ("int4", "e2m1"):
        g = F.grid_codes(grid)
        nib = F.element_nibbles(g, grid)
        assert nib.max() < 16
        np.testing.assert_array_equal(F.nibbles_to_values(nib, grid), g)
    assert list(F.element_nibbles(np.array([-8.0, -1.0, 7.0]), "int4")) == [8, 15, 7]
    assert list(F.element_nibbles(np.array([-6.0, 0.5, 0.0]), "e2m1")) == [15, 1, 0]


# --------------------------------------------------------------- scale sets

def test_fp16_table_is_all_positive_finite_halfs():
    vals, codes = F.scale_table("fp16")
    assert len(vals) == 31743
    assert vals[0] == 2.0 ** -24 and vals[-1] == 65504.0
    assert np.all(np.diff(vals) > 0)


def test_e4m3_table_matches_torch_float8():
    vals, codes = F.scale_table("e4m3")
    t = torch.arange(0, 256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = t.to(torch.float64).numpy()
    pos = np.unique(ref[np.isfinite(ref) & (ref > 0)])
    np.testing.assert_array_equal(vals, pos)
    assert vals[0] == 2.0 ** -9 and vals[-1] == 448.0 and len(vals) == 126
    assert F.encode_scale(np.array([1.0]), "e4m3")[0] == 0x38


def test_e8m0_table_is_powers_of_two():
    vals, codes = F.scale_table("e8m0")
    np.testing.assert_array_equal(vals, 2.0 ** np.arange(-127, 128))
    assert F.encode_scale(np.array([1.0]), "e8m0")[0] == 127


def _brute_nearest(x, fmt):
    vals, codes = F.scale_table(fmt)
    out = []
    for xi in x:
        d = np.abs(vals - xi)
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:
            if fmt == "e8m0":
                best = [best.max()]
            else:
                best = [i for i in best if codes[i] % 2 == 0]
        out.append(vals[best[0]])
    return np.array(out)


@pytest.mark.parametrize("fmt", ["fp16", "e4m3", "e8m0"])
def test_projection_is_nearest_legal_value(fmt):
    vals, _ = F.scale_table(fmt)
    sub = vals[:: max(1, len(vals) // 200)]
    mids = (vals[1:] + vals[:-1]) / 2
    mids = mids[:: max(1, len(mids) // 200)]
    x = np.concatenate([
        sub, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
        np.exp(RNG.uniform(np.log(vals[0]), np.log(vals[-1]), 500)),
        [vals[0] / 3, vals[-1] * 3],
    ])
    np.testing.assert_array_equal(F.project(x, fmt), _brute_nearest(x, fmt))


def test_fp16_projection_equals_numpy_rne_cast_in_range():
    x = np.exp(RNG.uniform(np.log(2.0 ** -24), np.log(65504.0), 20000))
    vals, _ = F.scale_table("fp16")
    mids = (vals[1:] + vals[:-1]) / 2
    x = np.concatenate([x, mids])
    np.testing.assert_array_equal(F.project(x, "fp16"),
                                  x.astype(np.float16).astype(np.float64))


def test_e4m3_projection_equals_torch_cast_in_range():
    vals, _ = F.scale_table("e4m3")
    mids = (vals[1:] + vals[:-1]) / 2
    x = np.concatenate([np.exp(RNG.uniform(np.log(2.0 ** -9), np.log(448.0), 5000)), mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(F.project(x, "e4m3"), ref)


def test_projection_clamps_and_saturates():
    assert F.project(np.array([1e-30]), "fp16")[0] == 2.0 ** -24
    assert F.project(np.array([1e9]), "fp16")[0] == 65504.0
    assert F.project(np.array([1e-30]), "e4m3")[0] == 2.0 ** -9
    assert F.project(np.array([470.0]), "e4m3")[0] == 448.0
    assert F.project(np.array([1e-60]), "e8m0")[0] == 2.0 ** -127
    # E8M0: x in [2^e, 2^(e+1)) goes up from 1.5 * 2^e on
    assert list(F.project(np.array([1.49999, 1.5, 2.9, 3.0]), "e8m0")) == [1, 2, 2, 4]


def test_projection_double_rounding_trap():
    # 1 + 2^-11 + 2^-40 is just above an fp16 midpoint: nearest is 1 + 2^-10.
    # Going through float32 first would land on the midpoint and round to 1.
    x = np.array([1 + 2.0 ** -11 + 2.0 ** -40])
    assert F.project(x, "fp16")[0] == 1 + 2.0 ** -10


@pytest.mark.parametrize("fmt", ["fp16", "e4m3", "e8m0"])
def test_encode_decode_round_trip(fmt):
    vals, codes = F.scale_table(fmt)
    enc = F.encode_scale(vals, fmt)
    np.testing.assert_array_equal(enc.astype(np.int64), codes)
    np.testing.assert_array_equal(F.decode_scale(enc, fmt), vals)
    if fmt == "fp16":
        np.testing.assert_array_equal(enc.view(np.float16).astype(np.float64), vals)
    with pytest.raises(ValueError):
        F.encode_scale(np.array([vals[1] * (1 + 1e-12)]), fmt)


# ------------------------------------------------------ 8-bit element grids

def test_int8_grid_rounds_half_even_and_clips_symmetric():
    # [SQuant tutorial] Ch. 2: symmetric int8 spans [-127, 127]
    x = np.array([-130.0, -127.5, -126.5, -0.5, 0.5, 1.5, 126.5, 127.4, 127.5, 300.0])
    assert list(F.round_int_grid(x, "int8")) == [-127, -127, -126, 0, 0, 2, 126, 127, 127, 127]
    assert F.grid_codes("int8")[0] == -127 and F.grid_codes("int8")[-1] == 127


def _e4m3_brute(x):
    vals = []
    codes = []
    for c in range(0x7F):                       # finite non-negative codes
        e, m = c >> 3, c & 7
        vals.append(m / 8 * 2.0 ** -6 if e == 0 else 2.0 ** (e - 7) * (1 + m / 8))
        codes.append(c)
    vals, codes = np.array(vals), np.array(codes)
    out = []
    for xi in x:
        ax = min(abs(xi), 448.0)
        d = np.abs(vals - ax)
        best = np.flatnonzero(d == d.min())
        pick = [i for i in best if codes[i] % 2 == 0] or list(best)
        v = vals[pick[0]]
        out.append(-v if xi < 0 else v)
    return np.array(out) + 0.0


def test_e4m3_elements_match_brute_force_and_torch():
    lv = F.e4m3_levels()
    mids = (lv[1:] + lv[:-1]) / 2
    x = np.concatenate([lv, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e3),
                        RNG.uniform(-460, 460, 3000), RNG.normal(0, 0.01, 1000)])
    x = np.concatenate([x, -x, [1e9, -1e9, 448.0, 449.0, 464.0]])
    got = F.round_e4m3(x)
    np.testing.assert_array_equal(got, _e4m3_brute(x))
    # torch's float8_e4m3fn cast rounds to nearest even within range
    inr = np.abs(x) <= 448.0
    xf = x[inr].astype(np.float32)
    ref = torch.from_numpy(xf).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(F.round_e4m3(xf.astype(np.float64)), ref + 0.0)
    assert not np.signbit(F.round_e4m3(np.array([-1e-9])))[0]


def test_8bit_code_round_trip():
    for grid in ("int8", "e4m3"):
        g = F.grid_codes(grid)
        c = F.element_codes(g, grid)
        np.testing.assert_array_equal(F.codes_to_values(c, grid), g)
        assert len(np.unique(c)) == len(g)
    assert list(F.element_codes(np.array([-127.0, -1.0, 5.0]), "int8")) == [0x81, 0xFF, 0x05]
    assert list(F.element_codes(np.array([1.0, -1.0, 448.0, 0.0]), "e4m3")) == [0x38, 0xB8, 0x7E, 0x00]
