"""End-to-end check of the factorization the solver feeds, a W4A4 reference
check ([DQ summary] §4.4 and App. I, [DQ repro] "Core equations":
X W^T ~= (X D_b) Q^T D_a, with the column scale folded into the activation
quantization and both operands in 4- or 8-bit codes with block scales).

The library's outputs -- packed weight codes, block scales a and column
scales b from the solver, packed activation codes and their scales from
dq_rescale_quantize_act -- are multiplied the way a W4A4 kernel would: per
block of G channels an integer (or E2M1) dot product of the codes, scaled by
the activation and weight block scales, accumulated in float32. That must
equal, up to float32 accumulation, the float64 product of the dequantized
operands, and it must approximate X W^T to within the quantization error.
No tuned GEMM is built: the product runs in plain torch float32 on the GPU.
"""

import numpy as np
import pytest
import torch

from calibration_free_bit_amd import dq, synth
from oracle import dualquant as D
from oracle import formats as F
from tests.gpu_util import decode_a, decode_b, oracle_fmt

pytestmark = pytest.mark.gpu

GRID_NAME = {dq.GRID_INT4: "int4", dq.GRID_E2M1: "e2m1", dq.GRID_INT8: "int8", dq.GRID_E4M3: "e4m3"}


def _code_table(fmt) -> torch.Tensor:
    n = 1 << fmt.code_bits
    return torch.tensor(F.codes_to_values(np.arange(n), GRID_NAME[fmt.grid]), dtype=torch.float32,
                        device="cuda")


def _unpack(packed: torch.Tensor, table: torch.Tensor, bits: int) -> torch.Tensor:
    if bits == 8:
        return table[packed.long()]
    lo = table[(packed & 0xF).long()]
    hi = table[(packed >> 4).long()]
    return torch.stack([lo, hi], dim=-1).reshape(packed.shape[0], packed.shape[1] * 2)


@pytest.mark.parametrize("name", ["int4_g64", "nvfp4_g16", "mxfp4_g32", "mxint8_g32", "mxfp8_g32"])
def test_w4a4_product_matches_factorization(name):
    fmt = dq.FORMATS[name]
    ofmt = oracle_fmt(fmt)
    G = fmt.group
    M, N, T = 256, 512, 64
    spec = synth.MatrixSpec(M, N, "normal", 0.02, 0.01, (20.0, 20.0), "bf16")
    Wm = synth.make_matrix(spec, 5)
    W = torch.from_numpy(Wm.data.view(np.int16)).cuda()
    s = dq.Solver(W, fmt)
    print(f"[case] w4a4 {name} {M}x{N} tokens {T}", flush=True)
    s.solve(10)
    Xh = synth.make_activations(T, N, 6)
    X = torch.from_numpy(Xh.view(np.int16)).cuda()
    xq = torch.empty((T, N * fmt.code_bits // 8), dtype=torch.uint8, device="cuda")
    xs = torch.empty((T, N // G), dtype=fmt.a_dtype, device="cuda")
    dq.rescale_quantize_act(s.p, X, T, N, s.b, xq, xs)
    torch.cuda.synchronize()

    table = _code_table(fmt)
    Qw = _unpack(s.packed, table, fmt.code_bits)           # [M, N] codes as values
    Qx = _unpack(xq, table, fmt.code_bits)                 # [T, N]
    a = torch.from_numpy(decode_a(s.a, fmt)).float().cuda()          # [M, N/G]
    sx = torch.from_numpy(decode_a(xs, fmt)).float().cuda()          # [T, N/G]

    # W4A4: per block, exact code dot products (small integers or halves, so
    # float32 is exact), then the two block scales, float32 accumulation
    Y = torch.zeros((T, M), dtype=torch.float32, device="cuda")
    for g in range(N // G):
        cs = slice(g * G, (g + 1) * G)
        P = Qx[:, cs].contiguous() @ Qw[:, cs].t().contiguous()       # [T, M]
        Y += P * sx[:, g:g + 1] * a[:, g][None, :]
    Y = Y.double().cpu().numpy()

    # float64 product of the dequantized operands: (s_x Xq) (D_a Q)^T
    a64, sx64 = decode_a(s.a, fmt), decode_a(xs, fmt)
    Qw64 = D.unpack_codes(s.packed.cpu().numpy(), ofmt)
    Qx64 = D.unpack_codes(xq.cpu().numpy(), ofmt)
    Xdq = Qx64 * np.repeat(sx64, G, axis=1)
    Wdq = Qw64 * np.repeat(a64, G, axis=1)
    Yref = Xdq @ Wdq.T
    scale = np.abs(Xdq) @ np.abs(Wdq).T
    assert np.all(np.abs(Y - Yref) <= 1e-5 * scale + 1e-30), np.max(np.abs(Y - Yref) / (scale + 1e-30))

    # and it approximates X W^T: the column scale cancels between the two
    # operands (X D_b times D_b^-1 W ~= D_a Q)
    b64 = decode_b(s.b)
    Xf = synth.bf16_to_f64(Xh)
    Wf = Wm.as_f64()
    Yexact = Xf @ Wf.T
    rel = np.linalg.norm(Yref - Yexact) / np.linalg.norm(Yexact)
    # the same product with the weights dequantized as D_a Q D_b and the
    # activations unscaled must agree with the factorized form exactly up to
    # the activation quantization: check the weight side alone
    What = D.reconstruct(a64, Qw64, b64, ofmt)
    rel_w = np.linalg.norm(Xf @ What.T - Yexact) / np.linalg.norm(Yexact)
    print(f"[w4a4 {name}] relative error of X W^T: W4A4 {rel:.4f}, weights only {rel_w:.4f}", flush=True)
    assert rel_w < rel < 0.5
