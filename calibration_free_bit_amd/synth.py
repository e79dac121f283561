"""Seeded synthetic inputs: LLM-shaped weight matrices and activations.

This module only draws random numbers and rounds them to the storage type.
It holds none of the quantizer's arithmetic, so both the float64 oracle and
the HIP library can be fed from it: the same uint16 bf16 bits (or float32
values) go to both sides.

Workloads stand in for the real checkpoints the DualQuant pages quantize
(Llama-3.1-8B and Qwen linear layers, [DQ summary] §5 and App. I): Gaussian
or Student-t bodies with a few outlier input channels (columns), which is
the structure that motivates the column scale ([DQ summary] §4.2; the
outlier problem in [RTN tutorial] "When RTN Fails").

Recipe: ``numpy.random.default_rng(seed)``
(PCG64); the body is drawn in float64 as one [M, N] array; then
``rng.choice(N, n_out, replace=False)`` picks n_out = round(frac * N) outlier
columns, then their factors are drawn (a uniform range, or a constant);
the columns are multiplied in float64; finally the matrix is rounded once,
to float32 or to bf16 (round-to-nearest-even, done on the float64 value
directly, no detour through float32).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


# ---------------------------------------------------------------- rounding

def bf16_bits(x) -> np.ndarray:
    """float64 -> bf16 bit patterns (uint16), round to nearest even.

    bf16 keeps 8 significant bits and float32's exponent range. Inputs must
    be zero or of magnitude within bf16's normal range (checked).
    """
    x = np.asarray(x, dtype=np.float64)
    nz = x != 0
    ax = np.abs(x[nz])
    if ax.size and (ax.min() < 2.0 ** -126 or ax.max() >= 2.0 ** 127):
        raise ValueError("value outside bf16's normal range")
    m, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    f = r.astype(np.float32)                 # exact: r has 8 significant bits
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values."""
    bits = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- matrices

@dataclass(frozen=True)
class MatrixSpec:
    rows: int
    cols: int
    dist: str                 # "normal" or "student_t4"
    std: float
    outlier_frac: float
    outlier_factor: tuple     # (lo, hi) uniform, or (c, c) constant
    dtype: str                # "bf16" or "f32"


@dataclass
class Matrix:
    spec: MatrixSpec
    seed: int
    data: np.ndarray          # uint16 bf16 bits or float32 values, [rows, cols]
    outlier_cols: np.ndarray

    def as_f64(self) -> np.ndarray:
        if self.spec.dtype == "bf16":
            return bf16_to_f64(self.data)
        return self.data.astype(np.float64)


def n_outliers(frac: float, cols: int) -> int:
    return int(round(frac * cols))


def make_matrix(spec: MatrixSpec, seed: int) -> Matrix:
    rng = np.random.default_rng(seed)
    shape = (spec.rows, spec.cols)
    if spec.dist == "normal":
        W = rng.normal(0.0, spec.std, size=shape)
    elif spec.dist == "student_t4":
        # Student-t with 4 degrees of freedom has std sqrt(2); rescale.
        W = rng.standard_t(4.0, size=shape) * (spec.std / np.sqrt(2.0))
    else:
        raise ValueError(spec.dist)
    n_out = n_outliers(spec.outlier_frac, spec.cols)
    cols = rng.choice(spec.cols, n_out, replace=False)
    lo, hi = spec.outlier_factor
    fac = rng.uniform(lo, hi, size=n_out) if hi != lo else np.full(n_out, float(lo))
    W[:, cols] *= fac[None, :]
    if spec.dtype == "bf16":
        data = bf16_bits(W)
    elif spec.dtype == "f32":
        data = W.astype(np.float32)
    else:
        raise ValueError(spec.dtype)
    return Matrix(spec, seed, data, np.sort(cols))


# ------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Workload:
    name: str
    spec: MatrixSpec
    fmt: str                  # "int4_g64" | "mxint4_g32" | "nvfp4_g16"
    iters: int
    seeds: tuple


#: Single-matrix workloads. Shapes are Llama-3.1-8B linears: q_proj
#: 4096x4096, gate/up 14336x4096, down 4096x14336 ([out, in] layout).
WORKLOADS = {
    "int4_g64_256x256_f32": Workload(
        "int4_g64_256x256_f32",
        MatrixSpec(256, 256, "normal", 0.02, 3 / 256, (20.0, 20.0), "f32"),
        "int4_g64", 10, (0, 1, 2)),
    "int4_g64_4096x4096_bf16": Workload(
        "int4_g64_4096x4096_bf16",
        MatrixSpec(4096, 4096, "normal", 0.02, 0.01, (10.0, 50.0), "bf16"),
        "int4_g64", 20, (0, 1, 2)),
    "mxint4_g32_14336x4096_bf16": Workload(
        "mxint4_g32_14336x4096_bf16",
        MatrixSpec(14336, 4096, "student_t4", 0.015, 0.005, (30.0, 30.0), "bf16"),
        "mxint4_g32", 20, (0, 1, 2)),
    "nvfp4_g16_4096x14336_bf16": Workload(
        "nvfp4_g16_4096x14336_bf16",
        MatrixSpec(4096, 14336, "normal", 0.01, 0.01, (25.0, 25.0), "bf16"),
        "nvfp4_g16", 20, (0, 1, 2)),
    # the gate/up projection shape of the Llama-3.1-8B set, with the set's
    # value recipe; seeds are the gate matrices of layers 0, 1 and 2
    "int4_g64_14336x4096_bf16": Workload(
        "int4_g64_14336x4096_bf16",
        MatrixSpec(14336, 4096, "normal", 0.02, 0.01, (20.0, 20.0), "bf16"),
        "int4_g64", 20, (4, 1004, 2004)),
    # the further MX formats, on the same 4096x4096 q_proj-shaped matrix
    "mxfp4_g32_4096x4096_bf16": Workload(
        "mxfp4_g32_4096x4096_bf16",
        MatrixSpec(4096, 4096, "normal", 0.02, 0.01, (10.0, 50.0), "bf16"),
        "mxfp4_g32", 20, (0, 1, 2)),
    "mxint8_g32_4096x4096_bf16": Workload(
        "mxint8_g32_4096x4096_bf16",
        MatrixSpec(4096, 4096, "normal", 0.02, 0.01, (10.0, 50.0), "bf16"),
        "mxint8_g32", 20, (0, 1, 2)),
    "mxfp8_g32_4096x4096_bf16": Workload(
        "mxfp8_g32_4096x4096_bf16",
        MatrixSpec(4096, 4096, "normal", 0.02, 0.01, (10.0, 50.0), "bf16"),
        "mxfp8_g32", 20, (0, 1, 2)),
}


@dataclass(frozen=True)
class ActWorkload:
    """Activation-side workload: X [tokens, cols] bf16 from make_activations,
    column scales from make_col_scales, quantized in ``fmt``."""
    name: str
    tokens: int
    cols: int
    fmt: str
    seed: int


#: Activation quantization with the column scales folded in: a prefill batch
#: of 8192 tokens entering the 4096-wide projections (q/k/v, gate/up) and
#: the 14336-wide down projection of Llama-3.1-8B.
ACT_WORKLOADS = {
    w.name: w for w in (
        ActWorkload("act_int4_g64_8192x4096_bf16", 8192, 4096, "int4_g64", 0),
        ActWorkload("act_mxint4_g32_8192x4096_bf16", 8192, 4096, "mxint4_g32", 0),
        ActWorkload("act_nvfp4_g16_8192x14336_bf16", 8192, 14336, "nvfp4_g16", 0),
    )
}

#: The 224 linear layers of Llama-3.1-8B: 32 layers x 7 projections,
#: [out, in] shapes. Seed of (layer l, projection p) is 1000*l + p.
LLAMA31_8B_PROJ = (("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096),
                   ("o", 4096, 4096), ("gate", 14336, 4096), ("up", 14336, 4096),
                   ("down", 4096, 14336))
LLAMA31_8B_LAYERS = 32


def llama_layer_specs():
    """[(layer, proj_index, name, MatrixSpec, seed)] for the full linear set."""
    out = []
    for l in range(LLAMA31_8B_LAYERS):
        for p, (name, M, N) in enumerate(LLAMA31_8B_PROJ):
            spec = MatrixSpec(M, N, "normal", 0.02, 0.01, (20.0, 20.0), "bf16")
            out.append((l, p, name, spec, 1000 * l + p))
    return out


def make_col_scales(cols: int, seed: int) -> np.ndarray:
    """fp16 bits of [cols] column inverse scales, log-uniform in [1/2, 2]
    (the spread of solved column scales around 1), rounded to nearest even.
    A stand-in for a solved b where only the activation side is measured."""
    rng = np.random.default_rng(seed)
    b = np.exp2(rng.uniform(-1.0, 1.0, size=cols))
    return b.astype(np.float16).view(np.uint16)


def make_activations(tokens: int, cols: int, seed: int, outlier_frac=0.01,
                     outlier_factor=20.0) -> np.ndarray:
    """bf16 bits of a [tokens, cols] activation matrix: N(0, 1) with a few
    outlier channels scaled by ``outlier_factor`` (the activation-outlier
    pattern of [RTN tutorial] "When RTN Fails")."""
    rng = np.random.default_rng(seed)
    X = rng.normal(0.0, 1.0, size=(tokens, cols))
    n_out = n_outliers(outlier_frac, cols)
    cols_out = rng.choice(cols, n_out, replace=False)
    X[:, cols_out] *= outlier_factor
    return bf16_bits(X)
