"""Number formats for the oracle: element grids, legal scale sets, projections.

TEST INFRASTRUCTURE ONLY (see the package docstring). Plain float64 numpy.

Sources
-------
* Element grids. [DQ summary] §3 "Quantization preliminaries": a value is
  divided by its scale, sent to the closest value the format can hold, and
  multiplied back; for integer grids that means rounding then clipping, for
  floating-point grids picking the closest of the (unevenly spaced) levels.
  The signed INT4
  codebook is [-8, 7] ([SQuant tutorial] Ch. 2 "Quantization from Scratch";
  [DQ repro] "Local reproduction"). The symmetric int8 range [-127, 127] is
  the one of the worked example in [SQuant tutorial] Ch. 2. NVFP4's element
  type is E2M1 (1 sign, 2 exponent, 1 mantissa bit), whose magnitudes are
  0, 0.5, 1, 1.5, 2, 3, 4, 6.
* Scale sets. [DQ summary] §3: MX formats use E8M0 (power-of-two) block
  scales; NVFP4 uses FP8 UE4M3 block scales; INT4 uses fp16 scales here.
  [DQ repro] "Core equations": the projection acts on the inverse scales,
  since a scale format can store only some positive reals.

Readings where the pages are silent:
* integer rounding ties go to the even integer (``np.rint``);
* E2M1 ties go to the level with the even encoding;
* a scale is projected onto its format's legal positive values by nearest
  linear distance -- the exact minimiser of the 1-D quadratic the update
  solves -- with ties to the even code for fp16 and E4M3 (IEEE-style
  round-half-even) and to the larger value for E8M0;
* values below the smallest legal positive value go to that value, values
  above the largest go to the largest (no zero, no infinity);
* "f32" is an unconstrained scale (the identity); it exists only so that
  the printed int8 example, which uses an unrounded scale, can be checked.
* 8-bit element grids ([DQ summary] §G.2 evaluates MXINT8 and MXFP8 without
  defining their elements): MXINT8 uses the symmetric int8 range
  [-127, 127] of [SQuant tutorial] Ch. 2; MXFP8 uses OCP E4M3FN elements
  (all finite E4M3 values), rounded to the nearest value with ties to the
  even code and saturated at 448.
"""

from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# Element grids
# --------------------------------------------------------------------------

#: Non-negative E2M1 magnitudes, in encoding order (code 0..7).
E2M1_LEVELS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

#: Integer grids: name -> (lowest code, highest code).
INT_GRIDS = {"int4": (-8, 7), "int8": (-127, 127)}

#: Largest magnitude of each grid; absmax init divides by this
#: ([DQ summary] §3: the symmetric scale is max|W| / qmax).
QMAX = {"int4": 7.0, "int8": 127.0, "e2m1": 6.0, "e4m3": 448.0}

#: Storage bits of one element code.
CODE_BITS = {"int4": 4, "e2m1": 4, "int8": 8, "e4m3": 8}


def round_int_grid(x: np.ndarray, grid: str) -> np.ndarray:
    """Round-and-clip onto an integer grid ([DQ summary] §3).

    Rounds to the nearest integer, ties to even, then clips to the grid's
    range. Returns float64 grid values.
    """
    lo, hi = INT_GRIDS[grid]
    return np.clip(np.rint(np.asarray(x, dtype=np.float64)), lo, hi)


def round_e2m1(x: np.ndarray) -> np.ndarray:
    """Nearest-level projection onto the E2M1 grid ([DQ summary] §3).

    The magnitude goes to the nearest of ``E2M1_LEVELS`` by linear distance
    (so anything above 6 goes to 6); at an exact midpoint between two levels
    the level whose encoding is even wins. The sign is kept; zero is +0.
    Returns float64 grid values.
    """
    x = np.asarray(x, dtype=np.float64)
    # every magnitude from 6 up has 6 as its nearest level; taking it there
    # first keeps the distances exact (far above 6, |x| - level would round
    # to the same float64 for every level)
    ax = np.minimum(np.abs(x), E2M1_LEVELS[-1])
    dist = np.abs(ax[..., None] - E2M1_LEVELS)          # [..., 8]
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best                                   # one or two True
    # among the nearest levels prefer an even code, else take the only one
    even = cand & (np.arange(8) % 2 == 0)
    idx = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    mag = E2M1_LEVELS[idx]
    return np.where(x < 0, -mag, mag) + 0.0               # -0 -> +0


def e4m3_levels() -> np.ndarray:
    """Non-negative E4M3FN element values in code order (code 0 is zero)."""
    vals, _ = _e4m3_table()
    return np.concatenate([[0.0], vals])


def round_e4m3(x: np.ndarray) -> np.ndarray:
    """Nearest-value projection onto the signed E4M3FN element grid.

    The magnitude goes to the nearest non-negative E4M3 value by linear
    distance, above 448 to 448; at an exact midpoint the value with the even
    code wins. The sign is kept; zero is +0. Returns float64 grid values.
    """
    x = np.asarray(x, dtype=np.float64)
    lv = e4m3_levels()
    ax = np.minimum(np.abs(x), lv[-1])
    hi = np.clip(np.searchsorted(lv, ax, side="left"), 1, len(lv) - 1)
    lo = hi - 1
    dlo, dhi = ax - lv[lo], lv[hi] - ax          # exact: neighbours within a factor of 2
    take_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    mag = np.where(take_hi, lv[hi], lv[lo])
    return np.where(x < 0, -mag, mag) + 0.0


def round_to_grid(x: np.ndarray, grid: str) -> np.ndarray:
    """The black-box element quantizer q of [DQ repro] "Core equations"."""
    if grid == "e2m1":
        return round_e2m1(x)
    if grid == "e4m3":
        return round_e4m3(x)
    return round_int_grid(x, grid)


def grid_codes(grid: str) -> np.ndarray:
    """All values of an element grid, ascending."""
    if grid == "e2m1":
        return np.unique(np.concatenate([-E2M1_LEVELS, E2M1_LEVELS]))
    if grid == "e4m3":
        lv = e4m3_levels()
        return np.unique(np.concatenate([-lv, lv]))
    lo, hi = INT_GRIDS[grid]
    return np.arange(lo, hi + 1, dtype=np.float64)


def tie_mask(x: np.ndarray, grid: str) -> np.ndarray:
    """True where x sits exactly on a rounding midpoint of the grid.

    Only those elements may legitimately round either way; every other
    element has one nearest grid value. Midpoints outside the clip range
    are not ties (both sides clip to the same code).
    """
    x = np.asarray(x, dtype=np.float64)
    g = grid_codes(grid)
    mids = (g[1:] + g[:-1]) / 2.0
    return np.isin(x, mids)


# --------------------------------------------------------------------------
# Legal scale sets
# --------------------------------------------------------------------------

def _fp16_table():
    codes = np.arange(1, 0x7C00, dtype=np.uint16)        # positive finite
    return codes.view(np.float16).astype(np.float64), codes.astype(np.int64)


def _e4m3_table():
    # OCP FP8 E4M3FN, sign bit clear: exponent bias 7, 3 mantissa bits,
    # exponent field 0 is subnormal (m/8 * 2^-6), code 0x7F is NaN.
    codes = np.arange(1, 0x7F, dtype=np.int64)
    e = codes >> 3
    m = codes & 7
    vals = np.where(e == 0, m / 8.0 * 2.0 ** -6, 2.0 ** (e - 7) * (1.0 + m / 8.0))
    return vals.astype(np.float64), codes


def _e8m0_table():
    # OCP E8M0: an 8-bit biased exponent, value 2^(code-127), code 255 is NaN.
    codes = np.arange(0, 255, dtype=np.int64)
    return np.ldexp(1.0, (codes - 127).astype(np.int64)), codes


_TABLES = {}


def scale_table(fmt: str):
    """(values ascending, native codes) of a scale format's legal values."""
    if fmt not in _TABLES:
        _TABLES[fmt] = {"fp16": _fp16_table, "e4m3": _e4m3_table,
                        "e8m0": _e8m0_table}[fmt]()
    return _TABLES[fmt]


def _nearest_index(x: np.ndarray, fmt: str) -> np.ndarray:
    """Index into ``scale_table(fmt)`` of the legal value nearest to x > 0."""
    vals, codes = scale_table(fmt)
    x = np.asarray(x, dtype=np.float64)
    hi = np.clip(np.searchsorted(vals, x, side="left"), 1, len(vals) - 1)
    lo = hi - 1
    # vals[lo] <= x <= vals[hi] inside the range; both differences are exact
    # in float64 because adjacent legal values are within a factor of two.
    dlo = x - vals[lo]
    dhi = vals[hi] - x
    if fmt == "e8m0":
        take_hi = dhi <= dlo                      # tie goes to the larger
    else:
        take_hi = (dhi < dlo) | ((dhi == dlo) & (codes[hi] % 2 == 0))
    idx = np.where(take_hi, hi, lo)
    idx = np.where(x <= vals[0], 0, idx)          # clamp below
    idx = np.where(x >= vals[-1], len(vals) - 1, idx)   # saturate above
    return idx


def project(x: np.ndarray, fmt: str) -> np.ndarray:
    """Projection Pi_F onto the legal positive scale values of ``fmt``.

    [DQ repro] "Core equations" and [DQ summary] App. B: every updated
    inverse scale is replaced by the closest value its format can hold.
    ``fmt`` is "fp16", "e8m0", "e4m3" or "f32" (identity).
    """
    x = np.asarray(x, dtype=np.float64)
    if fmt == "f32":
        return x.copy()
    vals, _ = scale_table(fmt)
    return vals[_nearest_index(x, fmt)]


def encode_scale(x: np.ndarray, fmt: str) -> np.ndarray:
    """Native storage code of legal scale values (uint16 fp16 bits, or the
    E8M0 / E4M3 byte). Raises if a value is not legal."""
    x = np.asarray(x, dtype=np.float64)
    vals, codes = scale_table(fmt)
    idx = np.searchsorted(vals, x)
    idx = np.clip(idx, 0, len(vals) - 1)
    if not np.all(vals[idx] == x):
        raise ValueError(f"value not representable in {fmt}")
    dt = np.uint16 if fmt == "fp16" else np.uint8
    return codes[idx].astype(dt)


def decode_scale(code: np.ndarray, fmt: str) -> np.ndarray:
    """Inverse of ``encode_scale``."""
    code = np.asarray(code).astype(np.int64)
    vals, codes = scale_table(fmt)
    lookup = np.full(int(codes.max()) + 1, np.nan)
    lookup[codes] = vals
    return lookup[code]


# --------------------------------------------------------------------------
# Element codes -> nibbles
# --------------------------------------------------------------------------

def element_nibbles(q: np.ndarray, grid: str) -> np.ndarray:
    """4-bit storage code of each grid value (uint8 in 0..15).

    INT4: two's complement. E2M1: sign bit 3, then the level's index 0..7
    (S.EE.M); zero is stored as +0.
    """
    q = np.asarray(q, dtype=np.float64)
    if grid == "int4":
        return (q.astype(np.int64) & 0xF).astype(np.uint8)
    if grid == "e2m1":
        idx = np.searchsorted(E2M1_LEVELS, np.abs(q))
        if not np.all(E2M1_LEVELS[np.clip(idx, 0, 7)] == np.abs(q)):
            raise ValueError("not an E2M1 value")
        sign = ((q < 0) & (q != 0)).astype(np.int64) << 3
        return (sign | idx).astype(np.uint8)
    raise ValueError(f"no 4-bit encoding for grid {grid}")


def element_codes(q: np.ndarray, grid: str) -> np.ndarray:
    """Storage code of each grid value: a nibble (see element_nibbles) for
    the 4-bit grids; a byte for the 8-bit ones -- int8 two's complement, or
    the E4M3FN byte (sign bit 7, zero stored as +0)."""
    q = np.asarray(q, dtype=np.float64)
    if CODE_BITS[grid] == 4:
        return element_nibbles(q, grid)
    if grid == "int8":
        return (q.astype(np.int64) & 0xFF).astype(np.uint8)
    if grid == "e4m3":
        lv = e4m3_levels()
        idx = np.searchsorted(lv, np.abs(q))
        if not np.all(lv[np.clip(idx, 0, len(lv) - 1)] == np.abs(q)):
            raise ValueError("not an E4M3 value")
        sign = ((q < 0) & (q != 0)).astype(np.int64) << 7
        return (sign | idx).astype(np.uint8)
    raise ValueError(grid)


def codes_to_values(code: np.ndarray, grid: str) -> np.ndarray:
    """Inverse of ``element_codes``."""
    if CODE_BITS[grid] == 4:
        return nibbles_to_values(code, grid)
    code = np.asarray(code).astype(np.int64) & 0xFF
    if grid == "int8":
        return np.where(code >= 128, code - 256, code).astype(np.float64)
    if grid == "e4m3":
        mag = e4m3_levels()[np.minimum(code & 0x7F, 126)]
        return np.where(code & 0x80, -mag, mag) + 0.0
    raise ValueError(grid)


def nibbles_to_values(nib: np.ndarray, grid: str) -> np.ndarray:
    """Inverse of ``element_nibbles``."""
    nib = np.asarray(nib).astype(np.int64) & 0xF
    if grid == "int4":
        return np.where(nib >= 8, nib - 16, nib).astype(np.float64)
    if grid == "e2m1":
        mag = E2M1_LEVELS[nib & 7]
        return np.where(nib & 8, -mag, mag) + 0.0
    raise ValueError(grid)
