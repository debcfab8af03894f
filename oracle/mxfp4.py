"""MXFP4 (32 E2M1 values under one power-of-two E8M0 scale) -- part of the oracle, so
TEST INFRASTRUCTURE like the rest of this package.

Ultralytics glossary "FP4":
  * §How FP4 works: MXFP4 is defined in the Open Compute Project Microscaling (MX)
    specification and groups 32 values under one 8-bit power-of-two scale (E8M0);
    an open format, supported by several vendors including AMD's MI350 series;
  * §FP4 for inference and training: native FP4 matrix units run MXFP4 on AMD
    Instinct MI350 accelerators.

The page does not say how the shared scale is chosen.  Reading taken here: the rule
of the OCP MX specification (v1.0, conversion to MX formats), which the page names:
  * shared exponent e = floor(log2(max_i |V_i|)) - 2, where 2 is the exponent of
    E2M1's largest value (6 = 1.5 * 2^2), clamped to E8M0's range [-127, 127]; a block
    of zeros gets e = -127;
  * scale byte = e + 127 (E8M0: value 2^(byte - 127); 0xFF, NaN, is never produced);
  * element codes: E2M1 round-to-nearest-even of V_i / 2^e, saturating at +-6 (since
    max |V| / 2^e lies in [4, 8), only values in (6, 8) saturate); zeros keep V_i's
    sign (nibble 8 for -0).
The dequantized value is E(P_i) * 2^e.  Layout: data [R, C/2] nibbles as for NVFP4
(element 2k in the low nibble of byte k), scales [R, C/32] bytes.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f32, e2m1_rne_code, e2m1_value
from .nvfp4 import pack_nibbles, unpack_nibbles

F32 = np.float32
BLOCK = 32
E2M1_EMAX = 2


def shared_exponent(amax: np.ndarray) -> np.ndarray:
    """e = floor(log2(amax)) - 2, clamped to [-127, 127]; -127 for amax == 0.  The
    floor of log2 comes from frexp (amax = m 2^x, m in [0.5, 1)), which is exact."""
    a = np.asarray(amax, dtype=np.float64)
    _, x = np.frexp(a)
    e = (x.astype(np.int64) - 1) - E2M1_EMAX
    e = np.clip(e, -127, 127)
    return np.where(a == 0, -127, e).astype(np.int64)


def quantize(x_bf16: np.ndarray) -> dict:
    """(R, C) bf16 bit patterns (uint16) or fp32 values, C % 32 == 0 ->
    {'data': (R, C/2) uint8, 'scales': (R, C/32) uint8}."""
    xb = np.asarray(x_bf16)
    x = bf16_bits_to_f32(xb) if xb.dtype == np.uint16 else np.asarray(xb, dtype=F32)
    R, C = x.shape
    assert C % BLOCK == 0, "cols must be a multiple of 32"
    blocks = x.astype(np.float64).reshape(R, C // BLOCK, BLOCK)
    amax = np.max(np.abs(blocks), axis=-1)
    e = shared_exponent(amax)
    v = blocks / np.exp2(e.astype(np.float64))[..., None]        # exact: power of two
    mag = e2m1_rne_code(np.abs(v))
    neg = np.signbit(blocks)
    codes = (mag | np.where(neg, 8, 0)).astype(np.uint8).reshape(R, C)
    return {"data": pack_nibbles(codes), "scales": (e + 127).astype(np.uint8)}


def dequantize(data: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """(R, C/2) nibbles and (R, C/32) E8M0 bytes -> (R, C) fp32 (exact)."""
    data = np.asarray(data, dtype=np.uint8)
    R, C = data.shape[0], data.shape[1] * 2
    vals = e2m1_value(unpack_nibbles(data)).reshape(R, C // BLOCK, BLOCK)
    e = np.asarray(scales, dtype=np.int64) - 127
    return (vals * np.exp2(e.astype(np.float64))[..., None]).reshape(R, C).astype(F32)


def operand_exact(data: np.ndarray, scales: np.ndarray, rows=None) -> np.ndarray:
    """Dequantized operand rows as fp64 (exact)."""
    data = np.asarray(data, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    if rows is not None:
        data, scales = data[rows], scales[rows]
    return dequantize(data, scales).astype(np.float64)


def gemm_ref64(a_data, a_scales, b_data, b_scales, rows=None, cols=None) -> np.ndarray:
    """Y = deq(A) deq(B)^T in fp64 for records A [M, K] and B [N, K] blocked along K
    (every product is exact in fp64; the sum rounds at fp64 precision)."""
    return operand_exact(a_data, a_scales, rows) @ operand_exact(b_data, b_scales, cols).T
