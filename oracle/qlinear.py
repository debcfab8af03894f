"""Reference for the simulated quantized linear forward Y = deq(Xq) . deq(Wq)^T.

Four Over Six documentation page, §Four Over Six: on hardware without native FP4
matrix operations (and on CPUs) the library simulates the quantized linear layer with
an FP32 matrix multiplication over the dequantized operands; §Training: the
quantized linear layer is a drop-in linear function.  Ultralytics glossary "FP4",
§FP4 for inference and training: FP4 products are accumulated in higher precision.

The reference here is exact up to fp64 rounding: every dequantized operand value is
E2M1 value times E4M3 value (at most 6 significant bits, exact in fp64) and the two
per-tensor scales are applied after the dot product:
    Y64[m, n] = t_x * t_w * sum_k (E*D)_x[m, k] * (E*D)_w[n, k]
Operands are in the row-wise layout, blocked along K: Xq [M, K], Wq [N, K] (the
PyTorch Linear weight layout [out, in]).

Backward (§Training: the quantized linear layer implements its backward pass): for
Y = X W^T and output gradient dY [M, N], dX = dY W and dW = dY^T X.  Each product is
formed from records blocked along its own inner dimension, which for W^T, dY^T and
X^T are the column-wise records (the quantizations of the transposes).
"""
from __future__ import annotations

import numpy as np

from .formats import e2m1_value, e4m3_value
from .nvfp4 import unpack_nibbles


def operand_exact(data: np.ndarray, scales: np.ndarray, rows=None) -> np.ndarray:
    """(E*D) for the selected rows as fp64 (exact), shape (len(rows), K)."""
    data = np.asarray(data, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    if rows is not None:
        data = data[rows]
        scales = scales[rows]
    R, K = data.shape[0], data.shape[1] * 2
    e = e2m1_value(unpack_nibbles(data)).reshape(R, K // 16, 16)
    dsc = e4m3_value(scales)[..., None]
    return (e * dsc).reshape(R, K)


def qlinear_ref64(x_data, x_scales, x_t, w_data, w_scales, w_t,
                  rows=None, cols=None) -> np.ndarray:
    """fp64 reference of Y (or of Y[rows][:, cols] when samples are given)."""
    ax = operand_exact(x_data, x_scales, rows)
    bw = operand_exact(w_data, w_scales, cols)
    return (float(x_t) * float(w_t)) * (ax @ bw.T)


def qlinear_bwd_ref64(dy=None, dyt=None, xt=None, wt=None):
    """fp64 references of the backward products.  Each argument is a record as a
    (data, scales, t) triple:
      dy : row-wise record of dY [M, N];      wt : record of W^T [K, N]
      dyt: record of dY^T [N, M];             xt : record of X^T [K, M]
    Returns (dX [M, K] = deq(dY) deq(W^T)^T, dW [N, K] = deq(dY^T) deq(X^T)^T); a
    product whose operands are missing is None."""
    dx = qlinear_ref64(*dy, *wt) if dy is not None and wt is not None else None
    dw = qlinear_ref64(*dyt, *xt) if dyt is not None and xt is not None else None
    return dx, dw
