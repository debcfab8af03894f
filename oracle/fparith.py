"""Correctly rounded fp32 fused multiply-add, for the oracle's error accumulation.

fma32(a, b, c) = RN_fp32(a*b + c) with a single rounding (IEEE 754 fusedMultiplyAdd,
round-to-nearest-even).  NumPy has no fp32 FMA, so it is built from exact fp64 pieces:
  * p = a*b is exact in fp64 (two 24-bit significands give at most 48 bits, and the
    fp32 exponent range squared stays inside fp64's normal range);
  * s = fl64(p + c) and its exact error r = (p + c) - s (Knuth's TwoSum);
  * f = RN_fp32(s) is the correct result unless s lies exactly on a midpoint between
    two fp32 neighbours and r != 0, in which case the sign of r decides the side (a
    midpoint of two fp32 values is representable in fp64, so no other case exists).
"""
from __future__ import annotations

import numpy as np


def fma32(a, b, c) -> np.ndarray:
    a64 = np.asarray(a, dtype=np.float32).astype(np.float64)
    b64 = np.asarray(b, dtype=np.float32).astype(np.float64)
    c64 = np.asarray(c, dtype=np.float32).astype(np.float64)
    p = a64 * b64
    with np.errstate(over="ignore", invalid="ignore"):
        s = p + c64
        bb = s - p
        r = (p - (s - bb)) + (c64 - bb)
        f = s.astype(np.float32)
        up = np.nextafter(f, np.float32(np.inf))
        dn = np.nextafter(f, np.float32(-np.inf))
        f64 = f.astype(np.float64)
        mid_up = (f64 + up.astype(np.float64)) * 0.5
        mid_dn = (f64 + dn.astype(np.float64)) * 0.5
    out = np.where((s == mid_up) & (r > 0), up, f)
    out = np.where((s == mid_dn) & (r < 0), dn, out)
    return out.astype(np.float32)
