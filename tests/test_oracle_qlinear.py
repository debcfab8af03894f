"""Pins for the oracle's qlinear reference (CPU only).

Four Over Six documentation page, §Four Over Six: without native FP4 matmuls the
quantized linear layer is simulated with an FP32 matrix multiplication of the
dequantized operands.  The oracle's fp64 reference must equal the exact product,
which Python integers compute here: every E2M1 x E4M3 value is an integer multiple of
2^-10, so Y / (t_x t_w) * 2^20 is an integer sum.
"""
import numpy as np

from oracle import formats as F
from oracle import nvfp4 as N
from oracle.qlinear import operand_exact, qlinear_ref64


def _q(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = F.f32_to_bf16_bits(rng.standard_normal((rows, cols)).astype(np.float32))
    return N.quantize(x, N.Config())


def test_qlinear_reference_is_exact_integer_product():
    qx, qw = _q(8, 64, 1), _q(6, 64, 2)
    y = qlinear_ref64(qx["row_data"], qx["row_scales"], qx["t"],
                      qw["row_data"], qw["row_scales"], qw["t"])
    ax = operand_exact(qx["row_data"], qx["row_scales"])
    bw = operand_exact(qw["row_data"], qw["row_scales"])
    ia = [[int(v * 1024) for v in row] for row in ax]
    ib = [[int(v * 1024) for v in row] for row in bw]
    assert np.all(ax * 1024 == np.round(ax * 1024))
    for m in range(8):
        for n in range(6):
            exact = sum(a * b for a, b in zip(ia[m], ib[n]))
            want = float(qx["t"]) * float(qw["t"]) * exact / 2.0 ** 20
            assert y[m, n] == want


def test_qlinear_reference_equals_dequantized_matmul():
    qx, qw = _q(32, 128, 3), _q(48, 128, 4)
    y = qlinear_ref64(qx["row_data"], qx["row_scales"], qx["t"],
                      qw["row_data"], qw["row_scales"], qw["t"])
    dx = N.dequantize(qx["row_data"], qx["row_scales"], qx["t"]).astype(np.float64)
    dw = N.dequantize(qw["row_data"], qw["row_scales"], qw["t"]).astype(np.float64)
    ref = dx @ dw.T           # fp32-rounded operands: agrees to fp32 relative precision
    assert np.linalg.norm(y - ref) <= 1e-6 * np.linalg.norm(y)


def test_qlinear_reference_sampled_rows_cols():
    qx, qw = _q(16, 64, 5), _q(32, 64, 6)
    full = qlinear_ref64(qx["row_data"], qx["row_scales"], qx["t"],
                         qw["row_data"], qw["row_scales"], qw["t"])
    rows, cols = np.array([3, 0, 15]), np.array([31, 2])
    part = qlinear_ref64(qx["row_data"], qx["row_scales"], qx["t"],
                         qw["row_data"], qw["row_scales"], qw["t"], rows, cols)
    assert np.array_equal(part, full[np.ix_(rows, cols)])
