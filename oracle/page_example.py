"""The worked example of block-size error on the Ultralytics glossary page "FP4",
§How FP4 works.

The page rounds a 4096-value tensor (N(0,1), torch seed 0, every 512th value times
20) onto the E2M1 grid three times: with one scale for the whole tensor, with one
scale per 32 values (the MXFP4 block size) and with one per 16 values (the NVFP4
block size).  Each scale is the block's largest magnitude divided by 6, values take
the nearest grid point (the first one on equal distance, i.e. the lower magnitude),
and the printed figure is the mean absolute error of the dequantized tensor.

This module restates that recipe in float32 NumPy, plus the same measurement for the
NVFP4 codec of ``nvfp4.py`` (E4M3 block scales under an FP32 tensor scale, 6-only
and 4/6 rules) so that the codec can be set beside the page's numbers.
"""
from __future__ import annotations

import numpy as np

from .formats import E2M1_GRID, f32_to_bf16_bits, bf16_bits_to_f32
from .nvfp4 import Config, dequantize, quantize

F32 = np.float32


def page_recipe_mae(x: np.ndarray, block: int) -> float:
    """Mean absolute error of the page's rule: scale = amax/6 per block (fp32),
    nearest grid point with ties to the lower magnitude, value = grid * sign * scale."""
    x = np.asarray(x, dtype=F32)
    blocks = x.reshape(-1, block)
    scale = (np.max(np.abs(blocks), axis=1, keepdims=True) / F32(6.0)).astype(F32)
    ratio = (np.abs(blocks) / scale).astype(F32)
    dist = np.abs(ratio[..., None] - E2M1_GRID.astype(F32)).astype(F32)
    idx = np.argmin(dist, axis=-1)                        # first minimum
    deq = (E2M1_GRID.astype(F32)[idx] * np.sign(blocks)).astype(F32)
    deq = (deq * scale).astype(F32)
    return float(np.mean(np.abs(deq.reshape(-1).astype(np.float64) - x.astype(np.float64))))


def page_recipe_mse(x: np.ndarray, block: int) -> float:
    x = np.asarray(x, dtype=F32)
    blocks = x.reshape(-1, block)
    scale = (np.max(np.abs(blocks), axis=1, keepdims=True) / F32(6.0)).astype(F32)
    ratio = (np.abs(blocks) / scale).astype(F32)
    idx = np.argmin(np.abs(ratio[..., None] - E2M1_GRID.astype(F32)), axis=-1)
    deq = (E2M1_GRID.astype(F32)[idx] * np.sign(blocks) * scale).astype(F32)
    return float(np.mean((deq.reshape(-1).astype(np.float64) - x.astype(np.float64)) ** 2))


def nvfp4_errors(x: np.ndarray, rule: str):
    """(MAE, MSE) of the NVFP4 codec on the same data, after rounding it to bf16,
    measured against the bf16-rounded input.  The tensor is laid out as one row."""
    xb = f32_to_bf16_bits(np.asarray(x, dtype=F32)).reshape(1, -1)
    q = quantize(xb, Config(rule=rule))
    deq = dequantize(q["row_data"], q["row_scales"], q["t"]).astype(np.float64)
    ref = bf16_bits_to_f32(xb).astype(np.float64)
    diff = deq - ref
    return float(np.mean(np.abs(diff))), float(np.mean(diff ** 2))
