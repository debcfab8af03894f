"""Random-sign 16-point Hadamard transform applied to each quantization block.

The Four Over Six documentation page (§Four Over Six) lists "the random Hadamard
transform" among the quantization options; the Ultralytics glossary "FP4" (§FP4 for
inference and training) says such transforms spread outliers.  Neither page fixes the
construction; readings taken here:
  * H16 is the Sylvester Hadamard matrix in natural order, normalised by 1/4 so that
    the transform is orthogonal;
  * one sign vector s (16 entries of +-1) per tensor: bit k of word 0 of
    Philox4x32-10(key = seed, counter = (0, 0, 0, 0)), set bit -> -1;
  * in fp32, each value is first multiplied by s_k/4 (exact for bf16 inputs), then
    the in-place fast Walsh-Hadamard butterflies run with strides 1, 2, 4, 8:
    (y_j, y_j+h) <- (y_j + y_j+h, y_j - y_j+h) for every j with (j & h) == 0;
  * the inverse (for dequantizing back to the original basis) uses that (H/4)^-1 =
    H/4 and S^-1 = S: multiply by 1/4, run the same butterflies, then apply the signs
    (all in fp32, in that order).
"""
from __future__ import annotations

import numpy as np

from .philox import philox4x32_10, split_seed


def rht_signs(seed: int) -> np.ndarray:
    """The tensor's 16 signs (+1.0 / -1.0) as float32."""
    w0 = int(philox4x32_10(np.zeros(4, dtype=np.uint64), split_seed(seed))[0])
    bits = np.array([(w0 >> k) & 1 for k in range(16)])
    return np.where(bits == 1, -1.0, 1.0).astype(np.float32)


def rht_blocks(blocks: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Transform each row of ``blocks`` (n, 16), float32 -> float32."""
    y = np.array(blocks, dtype=np.float32, copy=True)
    assert y.shape[-1] == 16
    y = y * (signs.astype(np.float32) * np.float32(0.25))
    for h in (1, 2, 4, 8):
        out = y.copy()
        for j in range(16):
            if j & h:
                continue
            a = y[..., j]
            b = y[..., j + h]
            out[..., j] = a + b
            out[..., j + h] = a - b
        y = out
    return y.astype(np.float32)


def irht_blocks(blocks: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Inverse transform of each row of ``blocks`` (n, 16), float32 -> float32."""
    return (rht_blocks(blocks, np.ones(16, dtype=np.float32)) * signs.astype(np.float32)
            ).astype(np.float32)
