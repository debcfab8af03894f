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
from oracle.qlinear import operand_exact, qlinear_bwd_ref64, qlinear_ref64


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


# ------------------------------------------------------------------ backward

def _grid_tensor(rows, cols, seed):
    """bf16 tensor whose entries are E2M1 grid values times 448, with a 6 * 448 in
    it: t = 1, and every 16-value block (row-wise, column-wise or 16x16) has a
    candidate that represents it exactly (max 6, 3 or 1.5 times 448 under the
    6-candidate; max 4, 2, 1 or 0.5 under the 4-candidate), so quantization under
    the 4/6 rule is lossless."""
    rng = np.random.default_rng(seed)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    v = grid[rng.integers(0, 8, (rows, cols))] * rng.choice([-1.0, 1.0], (rows, cols))
    v[rng.integers(rows), rng.integers(cols)] = 6.0
    return v * 448.0


def _records(x64, cfg):
    q = N.quantize(F.f32_to_bf16_bits(x64.astype(np.float32)), cfg)
    out = {}
    for lay in ("row", "col"):
        if f"{lay}_data" in q:
            out[lay] = (q[f"{lay}_data"], q[f"{lay}_scales"], q["t"])
    return out


def test_grid_tensors_quantize_losslessly():
    x = _grid_tensor(48, 64, 11)
    for cfg in (N.Config(cols_out=True), N.Config(cols_out=True, block="2d")):
        r = _records(x, cfg)
        assert float(r["row"][2]) == 1.0
        assert np.array_equal(N.dequantize(*r["row"]).astype(np.float64), x)
        assert np.array_equal(N.dequantize(*r["col"]).astype(np.float64), x.T)


def test_backward_references_equal_exact_gradients():
    """On losslessly quantized operands the references are the exact gradients of a
    linear layer: dX = dY W, dW = dY^T X (integers, so fp64 sums are exact)."""
    M, Nn, K = 48, 80, 64
    x, w, dy = _grid_tensor(M, K, 1), _grid_tensor(Nn, K, 2), _grid_tensor(M, Nn, 3)
    cfg = N.Config(cols_out=True)
    rx, rw, rdy = _records(x, cfg), _records(w, cfg), _records(dy, cfg)
    dx, dw = qlinear_bwd_ref64(dy=rdy["row"], dyt=rdy["col"], xt=rx["col"], wt=rw["col"])
    assert np.array_equal(dx, dy @ w)
    assert np.array_equal(dw, dy.T @ x)
    # a transposed operand is caught: dY W^T has the wrong shape, dY^T X^T too
    assert dx.shape == (M, K) and dw.shape == (Nn, K)


def test_backward_hadamard_cancels_along_the_inner_dimension():
    """dW from the column-wise records of dY and X, both with the same random-sign
    Hadamard transform along M, approximates dY^T X (the transform is orthogonal);
    with different seeds it does not."""
    rng = np.random.default_rng(5)
    M, Nn, K = 256, 48, 32
    x = rng.standard_normal((M, K))
    dy = rng.standard_normal((M, Nn))
    exact = dy.T @ x

    def rel(seed_dy, seed_x):
        qd = N.quantize(F.f32_to_bf16_bits(dy.astype(np.float32)),
                        N.Config(rows_out=False, cols_out=True, hadamard=True,
                                 hadamard_seed=seed_dy))
        qx = N.quantize(F.f32_to_bf16_bits(x.astype(np.float32)),
                        N.Config(rows_out=False, cols_out=True, hadamard=True,
                                 hadamard_seed=seed_x))
        _, dw = qlinear_bwd_ref64(dyt=(qd["col_data"], qd["col_scales"], qd["t"]),
                                  xt=(qx["col_data"], qx["col_scales"], qx["t"]))
        return np.linalg.norm(dw - exact) / np.linalg.norm(exact)

    assert rel(7, 7) < 0.15
    assert rel(7, 8) > 0.5
