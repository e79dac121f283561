"""The DualQuant dual-scale quantizer solved by block-coordinate descent.

TEST INFRASTRUCTURE ONLY (see the package docstring). Plain float64 numpy;
no blocking, fusion or reordering beyond what the pages state.

Notation ([DQ repro] "Core equations"; [DQ summary] §4.2):
  W      [M, N] weight (nn.Linear layout: row i = output channel,
         column j = input channel), held exactly as float64.
  G      block size: groups of G contiguous elements along each row
         ([DQ summary] §3, block-wise quantization).
  a      [M, N/G] row/block inverse scales (a = alpha^-1).
  b      [N] column inverse scales (b = beta^-1).
  Q      codes, Q_ij = q(W_ij / (a_i,g(j) * b_j)), q the black-box element
         quantizer of the format.
  W ~= D_a Q D_b, i.e. W_ij ~= a_i,g(j) * Q_ij * b_j.

The iteration ([DQ repro] "Core equations" and the flowchart under
"Background and contribution"; [DQ summary] §4.3, App. A.1, A.2, App. B):
with the codes fixed, each outer inverse scale has its own 1-D least-squares
problem with a closed-form solution,
  a_i <- Pi_Fa( sum_j W_ij R_ij / sum_j R_ij^2 ),   R = Q D_b,
  b_j <- Pi_Fb( sum_i W_ij S_ij / sum_i S_ij^2 ),   S = D_a Q,
the result is projected onto the format's legal scale values, the inner
copies (the ones that assign codes) are synchronized with the outer ones,
and the codes are requantized after the row update and again after the
column update. A slice whose codes are all zero gets scale 1.

Readings where the pages are silent:
* one copy of each scale: synchronizing the inner copy right after each
  projection makes the two copies equal whenever codes are assigned;
* a_i is per (row, block): the sums run over the G columns of the block;
  b_j runs over all M rows of the whole matrix;
* initialization is absmax RTN: a = Pi_Fa(absmax / qmax) per block (1 for
  an all-zero block), b = 1;
* exactly T iterations, each (row update, requant, column update, requant),
  after one initial requant; no early stop.

Float64 is exact here up to summation order: W (bf16 or fp32) converts
exactly, every product W*Q*b, (Q*b)^2, W*a*Q, (a*Q)^2 fits in 53 bits, a*b is
exact, and W / (a*b) is one correctly rounded division, so every rounding
tie of the element quantizer is decided on the exact value.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import formats as F


@dataclass(frozen=True)
class Format:
    """A black-box quantization format.

    grid  -- element grid: "int4" [-8, 7], "e2m1", or "int8" [-127, 127]
    group -- block size G along each row
    a_fmt -- legal set of the block scales: "fp16", "e8m0", "e4m3", "f32"
    b_fmt -- legal set of the column scales
    """
    grid: str
    group: int
    a_fmt: str
    b_fmt: str = "fp16"

    @property
    def qmax(self) -> float:
        return F.QMAX[self.grid]


#: Formats named by [DQ summary] §3 and §5: INT4 with G=64 (the packed
#: deployment of App. I), MXINT4 (G=32, E8M0 scales), NVFP4 (E2M1, G=16,
#: UE4M3 scales). Column scales are fp16.
INT4_G64 = Format("int4", 64, "fp16", "fp16")
MXINT4_G32 = Format("int4", 32, "e8m0", "fp16")
NVFP4_G16 = Format("e2m1", 16, "e4m3", "fp16")
MXFP4_G32 = Format("e2m1", 32, "e8m0", "fp16")
#: The 8-bit MX formats of [DQ summary] §G.2 (elements: see oracle.formats).
MXINT8_G32 = Format("int8", 32, "e8m0", "fp16")
MXFP8_G32 = Format("e4m3", 32, "e8m0", "fp16")
FORMATS = {"int4_g64": INT4_G64, "mxint4_g32": MXINT4_G32, "nvfp4_g16": NVFP4_G16,
           "mxfp4_g32": MXFP4_G32, "mxint8_g32": MXINT8_G32, "mxfp8_g32": MXFP8_G32}


def _check(W: np.ndarray, fmt: Format) -> np.ndarray:
    W = np.asarray(W, dtype=np.float64)
    if W.ndim != 2 or W.shape[1] % fmt.group:
        raise ValueError("W must be [M, N] with N a multiple of the group size")
    return W


def expand_blocks(a: np.ndarray, group: int) -> np.ndarray:
    """[M, N/G] block scales -> [M, N], each repeated over its G columns."""
    return np.repeat(np.asarray(a, dtype=np.float64), group, axis=1)


def block_sums(x: np.ndarray, group: int) -> np.ndarray:
    """Sum of each row's groups of G contiguous columns: [M, N] -> [M, N/G]."""
    M, N = x.shape
    return x.reshape(M, N // group, group).sum(axis=2)


def scaled(W, a, b, fmt: Format) -> np.ndarray:
    """x_ij = W_ij / (a_i,g(j) * b_j), one correctly rounded division."""
    return W / (expand_blocks(a, fmt.group) * np.asarray(b, dtype=np.float64)[None, :])


def quantize(W, a, b, fmt: Format) -> np.ndarray:
    """Requantization Q = q(W / (a b)) ([DQ repro] "Core equations")."""
    return F.round_to_grid(scaled(W, a, b, fmt), fmt.grid)


def code_ties(W, a, b, fmt: Format) -> np.ndarray:
    """Elements whose scaled value is exactly on a rounding midpoint."""
    return F.tie_mask(scaled(W, a, b, fmt), fmt.grid)


def init_rtn(W, fmt: Format):
    """Absmax round-to-nearest initialization.

    [DQ summary] §3: the symmetric scale is max|W| / qmax, and block-wise
    quantization gives every group of G contiguous row elements its own
    scale; §5.3: initialization uses format-native row absmax scales.
    [RTN tutorial] "Absmax (Symmetric) Quantization". The column scales
    start at 1. A block whose absmax is 0 gets scale 1.
    Returns (a [M, N/G], b [N]).
    """
    W = _check(W, fmt)
    M, N = W.shape
    amax = np.abs(W).reshape(M, N // fmt.group, fmt.group).max(axis=2)
    a = np.where(amax > 0, F.project(amax / fmt.qmax, fmt.a_fmt), 1.0)
    b = np.ones(N)
    return a, b


def init_colnorm(W, fmt: Format):
    """Initialization from per-column L1 norms and format-native row absmax.

    [DQ summary] §5.3: the starting point combines format-native row absmax
    scales with per-column L1-norm scales; the page gives no formula.
    Reading: the column inverse scale is its column's
    mean absolute value projected onto F_b, b_j = Pi_Fb(sum_i |W_ij| / M)
    (1 for an all-zero column), and the block scales are the absmax
    initialization applied to W D_b^-1,
    a_ig = Pi_Fa(max_{j in g} |W_ij / b_j| / qmax) (1 for a zero block).
    Returns (a [M, N/G], b [N]).
    """
    W = _check(W, fmt)
    M = W.shape[0]
    colmean = np.abs(W).sum(axis=0) / M
    b = np.where(colmean > 0, F.project(np.where(colmean > 0, colmean, 1.0), fmt.b_fmt), 1.0)
    a, _ = init_rtn(W / b[None, :], fmt)
    return a, b


def update_a(W, Q, b, fmt: Format) -> np.ndarray:
    """Closed-form row/block update with the codes and b fixed.

    [DQ repro] "Core equations": a_i <- Pi_Fa(sum_j W_ij R_ij / sum_j R_ij^2)
    with R = Q D_b; the sums run over the block's G columns. An all-zero
    code slice (den = 0) gets scale 1.
    """
    W = _check(W, fmt)
    R = Q * np.asarray(b, dtype=np.float64)[None, :]
    num = block_sums(W * R, fmt.group)
    den = block_sums(R * R, fmt.group)
    ratio = num / np.where(den > 0, den, 1.0)
    return np.where(den > 0, F.project(np.where(den > 0, ratio, 1.0), fmt.a_fmt), 1.0)


def update_b(W, Q, a, fmt: Format) -> np.ndarray:
    """Closed-form column update with the codes and a fixed.

    [DQ repro] "Core equations": b_j <- Pi_Fb(sum_i W_ij S_ij / sum_i S_ij^2)
    with S = D_a Q; the sums run over all M rows. An all-zero code column
    gets scale 1.
    """
    W = _check(W, fmt)
    S = expand_blocks(a, fmt.group) * Q
    num = (W * S).sum(axis=0)
    den = (S * S).sum(axis=0)
    ratio = num / np.where(den > 0, den, 1.0)
    return np.where(den > 0, F.project(np.where(den > 0, ratio, 1.0), fmt.b_fmt), 1.0)


def reconstruct(a, Q, b, fmt: Format) -> np.ndarray:
    """W_hat = D_a Q D_b ([DQ repro] "Core equations")."""
    return expand_blocks(a, fmt.group) * Q * np.asarray(b, dtype=np.float64)[None, :]


def sse(W, a, Q, b, fmt: Format) -> float:
    """Sum of squared reconstruction errors."""
    return float(((np.asarray(W, dtype=np.float64) - reconstruct(a, Q, b, fmt)) ** 2).sum())


@dataclass
class Solution:
    a: np.ndarray
    b: np.ndarray
    Q: np.ndarray
    #: SSE after init and after every sub-step, in the order
    #: init, (R, Q1, C, Q2) x T -- filled when history=True
    sse: list = field(default_factory=list)
    #: number of codes that changed in each iteration (Q at the end of the
    #: iteration against Q at its start) -- filled when history=True
    changed: list = field(default_factory=list)


def solve(W, fmt: Format, iters: int, a=None, b=None, history: bool = False) -> Solution:
    """Run the BCD solver for exactly ``iters`` iterations.

    Flow of [DQ repro] (flowchart and "Core equations"): initial requant,
    then per iteration: fixed-code row update -> project and synchronize ->
    requantize -> fixed-code column update -> project -> requantize.
    Starting scales default to ``init_rtn``; passing (a, b) resumes a
    previous solve (the state of the solver is exactly (a, b)).
    """
    W = _check(W, fmt)
    if a is None:
        a, b = init_rtn(W, fmt)
    a = np.asarray(a, dtype=np.float64).copy()
    b = np.asarray(b, dtype=np.float64).copy()
    Q = quantize(W, a, b, fmt)
    out = Solution(a, b, Q)
    if history:
        out.sse.append(sse(W, a, Q, b, fmt))
    for _ in range(iters):
        Q_start = Q
        a = update_a(W, Q, b, fmt)                       # (R)
        if history:
            out.sse.append(sse(W, a, Q, b, fmt))
        Q = quantize(W, a, b, fmt)                       # (Q1)
        if history:
            out.sse.append(sse(W, a, Q, b, fmt))
        b = update_b(W, Q, a, fmt)                       # (C)
        if history:
            out.sse.append(sse(W, a, Q, b, fmt))
        Q = quantize(W, a, b, fmt)                       # (Q2)
        if history:
            out.sse.append(sse(W, a, Q, b, fmt))
            out.changed.append(int((Q != Q_start).sum()))
    out.a, out.b, out.Q = a, b, Q
    return out


def iteration_stats(W, fmt: Format, iters: int, a=None, b=None) -> np.ndarray:
    """Convergence diagnostics of a solve, one row per state.

    [DQ summary] §5.3 and the convergence figure of App. B follow the
    normalized reconstruction error and the share of codes that change from
    one iteration to the next. Row k (k = 0 .. iters) describes the state
    after k iterations (row 0: the starting state): the squared
    reconstruction error sum (W - D_a Q D_b)^2, sum W^2 (their ratio is the
    normalized error) and the number of codes that differ from those of
    state k - 1 (0 in row 0). Returns float64 [iters + 1, 3].
    """
    W = _check(W, fmt)
    sol = solve(W, fmt, iters, a, b, history=True)
    out = np.zeros((iters + 1, 3))
    out[:, 0] = sol.sse[0::4]          # the start, then the end of every iteration
    out[:, 1] = float((W * W).sum())
    out[1:, 2] = sol.changed
    return out


# --------------------------------------------------------------------------
# Emit: packed codes and native scale encodings
# --------------------------------------------------------------------------

def pack_codes(Q, fmt: Format) -> np.ndarray:
    """Codes in storage form. 4-bit grids: two codes per byte, low nibble =
    even column, [M, N/2] uint8; 8-bit grids: one code per byte, [M, N].

    [DQ summary] App. I packs INT4 weights offline for deployment. INT4 codes
    are two's complement; E2M1 codes are sign + level index; int8 is two's
    complement and E4M3 the FP8 byte.
    """
    codes = F.element_codes(Q, fmt.grid)
    if F.CODE_BITS[fmt.grid] == 8:
        return codes.astype(np.uint8)
    if codes.shape[1] % 2:
        raise ValueError("packing needs an even number of columns")
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed, fmt: Format) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    if F.CODE_BITS[fmt.grid] == 8:
        return F.codes_to_values(packed, fmt.grid)
    lo = F.nibbles_to_values(packed & 0xF, fmt.grid)
    hi = F.nibbles_to_values(packed >> 4, fmt.grid)
    out = np.empty((packed.shape[0], packed.shape[1] * 2))
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def footprint_bytes(M: int, N: int, fmt: Format):
    """Bytes of the emitted artefacts: (packed codes, a, b)."""
    a_bytes = 2 if fmt.a_fmt == "fp16" else 1
    return M * N * F.CODE_BITS[fmt.grid] // 8, M * (N // fmt.group) * a_bytes, N * 2


# --------------------------------------------------------------------------
# Activation side (inference factorization)
# --------------------------------------------------------------------------

def rescale_quantize_act(X, b, fmt: Format):
    """Column-scale fold plus per-token block quantization of activations.

    [DQ summary] §4.4: at inference the column scale rescales activations
    before format-native row-wise quantization (the multiply lives inside
    the activation-quantization kernel); [DQ repro] "Core equations":
    X W^T ~= (X D_beta^-1) Q^T D_alpha^-1 = (X D_b) Q^T D_a.
    Each token row of X D_b is quantized in blocks of G contiguous channels
    with absmax scales projected to the block-scale format (scale 1 for an
    all-zero block).
    Returns (codes [T, N] as grid values, scales [T, N/G]).
    """
    X = np.asarray(X, dtype=np.float64)
    Xs = X * np.asarray(b, dtype=np.float64)[None, :]
    s, _ = init_rtn(Xs, fmt)
    return quantize(Xs, s, np.ones(X.shape[1]), fmt), s
