"""The worked example of block-size error on the Ultralytics glossary page "FP4",
§How FP4 works -- TEST INFRASTRUCTURE (part of the oracle).

The section rounds a 4096-value tensor onto the E2M1 grid three times, with one scale
for the whole tensor, with one scale per 32 values (MXFP4's block size) and with one
per 16 values (NVFP4's), and prints the mean absolute error of each.  In its words,
a block's scale is the one that maps the block's largest magnitude to 6, the largest
E2M1 value, and every value becomes the nearest grid point of value / scale.  Its
example picks the first of two equally distant grid points, i.e. the smaller
magnitude; ``formats.e2m1_nearest_lower_code`` states that rule.

``block_scale_mae`` restates the measurement with the oracle's own pieces, in fp32
like the page; ``nvfp4_errors`` takes the same measurement for the NVFP4 codec of
``nvfp4.py`` (E4M3 block scales under an FP32 tensor scale, 6-only and 4/6 rules) so
that the codec can be set beside the page's numbers.
"""
from __future__ import annotations

import numpy as np

from .formats import E2M1_GRID, bf16_bits_to_f32, e2m1_nearest_lower_code, f32_to_bf16_bits
from .nvfp4 import Config, dequantize, quantize

F32 = np.float32


def block_scale_mae(x: np.ndarray, block: int) -> float:
    """Mean absolute error of one max -> 6 scale per ``block`` consecutive values.

    For each block: s = RN32(max|x| / 6); each value's magnitude is divided by s in
    fp32 and mapped to its nearest grid point (ties to the smaller magnitude); the
    reconstruction is the grid value times s with the value's sign, in fp32.  The
    error is averaged over all values in fp64.  A block of zeros reconstructs as
    zeros (no scale is needed for it)."""
    x = np.asarray(x, dtype=F32).reshape(-1)
    assert x.size % block == 0
    err = np.empty(x.size, dtype=np.float64)
    for b0 in range(0, x.size, block):
        v = x[b0:b0 + block]
        s = F32(np.max(np.abs(v)) / F32(6.0))
        if s == 0:
            rec = np.zeros(block, dtype=F32)
        else:
            code = e2m1_nearest_lower_code((np.abs(v) / s).astype(F32))
            rec = (E2M1_GRID[code].astype(F32) * s).astype(F32)
            rec = np.where(np.signbit(v), -rec, rec)
        err[b0:b0 + block] = np.abs(rec.astype(np.float64) - v.astype(np.float64))
    return float(np.mean(err))


def nvfp4_errors(x: np.ndarray, rule: str):
    """(MAE, MSE) of the NVFP4 codec on the same data, after rounding it to bf16,
    measured against the bf16-rounded input.  The tensor is laid out as one row."""
    xb = f32_to_bf16_bits(np.asarray(x, dtype=F32)).reshape(1, -1)
    q = quantize(xb, Config(rule=rule))
    deq = dequantize(q["row_data"], q["row_scales"], q["t"]).astype(np.float64)
    ref = bf16_bits_to_f32(xb).astype(np.float64)
    diff = deq - ref
    return float(np.mean(np.abs(diff))), float(np.mean(diff ** 2))
