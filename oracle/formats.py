"""Number formats: E2M1 (FP4), E4M3 (FP8 scale) and bfloat16, as plain definitions.

Ultralytics glossary "FP4", opening section: E2M1 has one sign, two exponent and one
mantissa bit and represents exactly 0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6.
Same page, §How FP4 works: the NVFP4 block scale is an FP8 E4M3 number.

Readings taken here (the pages give only the value sets):
  * E2M1 code assignment follows the usual float layout with exponent bias 1:
    magnitude codes 0..7 <-> 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign.
  * E4M3 is the OCP "FN" variant: bias 7, largest finite value 448, no infinities,
    code 0x7F/0xFF is NaN.  The per-tensor constant 448*6 fixes 448 as the maximum.
  * Rounding is round-to-nearest with ties to the even code, and saturates at the
    largest finite value (6 for E2M1, 448 for E4M3).

All encoders here are brute force over the value set (nearest value, computed with
exact fp64 distances), which is the plain definition of round-to-nearest-even.
"""
from __future__ import annotations

import numpy as np

# E2M1 magnitudes by code (bit 3 of the nibble is the sign).
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_value(nibble: np.ndarray) -> np.ndarray:
    """Signed fp64 value of 4-bit codes; code 8 is -0.0."""
    nib = np.asarray(nibble).astype(np.int64)
    mag = E2M1_GRID[nib & 7]
    return np.where((nib & 8) != 0, -mag, mag)


def _nearest(values: np.ndarray, table: np.ndarray, ties: str) -> np.ndarray:
    """Index of the nearest entry of the increasing ``table`` to each value (fp64
    exact distances).  An exact tie between two entries goes to the even index
    (``ties="even"``) or to the lower entry (``ties="lower"``); values beyond the last
    entry map to the last entry (saturation)."""
    v = np.asarray(values, dtype=np.float64)
    hi = np.searchsorted(table, v, side="left")          # table[hi-1] < v <= table[hi]
    hi = np.clip(hi, 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    d_lo = np.abs(v - table[lo])
    d_hi = np.abs(table[hi] - v)
    if ties == "even":
        tie_hi = hi % 2 == 0
    elif ties == "lower":
        tie_hi = np.zeros(v.shape, dtype=bool)
    else:
        raise ValueError(ties)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & tie_hi)
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(v >= table[-1], len(table) - 1, idx)
    return idx.astype(np.int64)


def _nearest_even(values: np.ndarray, table: np.ndarray) -> np.ndarray:
    return _nearest(values, table, "even")


def e2m1_rne_code(magnitude: np.ndarray) -> np.ndarray:
    """Magnitude code (0..7) of round-to-nearest-even of |v| onto the E2M1 grid,
    saturating at 6.  Input must be finite and >= 0."""
    m = np.asarray(magnitude, dtype=np.float64)
    assert np.all(m >= 0) and np.all(np.isfinite(m))
    return _nearest_even(m, E2M1_GRID).astype(np.uint8)


def e2m1_nearest_lower_code(magnitude: np.ndarray) -> np.ndarray:
    """Magnitude code (0..7) of the nearest E2M1 value to |v|, an exact tie going to
    the smaller magnitude (0.25 -> 0, 0.75 -> 0.5, 1.75 -> 1.5, 3.5 -> 3, ...),
    saturating at 6.  This is the rule of the worked example on the Ultralytics
    glossary page "FP4" (§How FP4 works), which picks the first grid point at the
    smallest distance.  Input must be finite and >= 0."""
    m = np.asarray(magnitude, dtype=np.float64)
    assert np.all(m >= 0) and np.all(np.isfinite(m))
    return _nearest(m, E2M1_GRID, "lower").astype(np.uint8)


# ---- E4M3 (OCP FN) ---------------------------------------------------------------

def _e4m3_table() -> np.ndarray:
    """Values of the 127 non-negative finite codes 0x00..0x7E, from the bit layout:
    exponent field e (4 bits, bias 7), mantissa m (3 bits);
    e == 0: m * 2^-9 (subnormal); otherwise 2^(e-7) * (1 + m/8)."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(m * 2.0 ** -9)
        else:
            vals.append(2.0 ** (e - 7) * (1.0 + m / 8.0))
    return np.array(vals, dtype=np.float64)


E4M3_TABLE = _e4m3_table()
E4M3_MAX = 448.0


def e4m3_value(code: np.ndarray) -> np.ndarray:
    """Value (fp64, exact) of non-negative E4M3 codes 0x00..0x7E."""
    c = np.asarray(code).astype(np.int64)
    assert np.all((c >= 0) & (c <= 0x7E))
    return E4M3_TABLE[c]


def e4m3_rne_sat(r: np.ndarray) -> np.ndarray:
    """E4M3 code of round-to-nearest-even of r >= 0 (subnormals kept), saturating to
    448 (0x7E) for every r above the largest finite value.  +inf maps to 0x7E."""
    v = np.asarray(r, dtype=np.float64)
    assert np.all(v >= 0) and not np.any(np.isnan(v))
    v = np.minimum(v, 2.0 * E4M3_MAX)           # +inf -> a value that saturates
    return _nearest_even(v, E4M3_TABLE).astype(np.uint8)


# ---- bfloat16 ----------------------------------------------------------------------

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 values (exact: bf16 is the upper half
    of an fp32 pattern)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even), returned as uint16 bit
    patterns.  The two bf16 neighbours of x are the truncation of its fp32 pattern and
    the next pattern away from zero; pick the nearer (exact fp64 distances) and, on a
    tie, the one with an even last bit.  Finite inputs only."""
    x = np.asarray(x, dtype=np.float32)
    assert np.all(np.isfinite(x))
    u = x.view(np.uint32)
    down = u & np.uint32(0xFFFF0000)
    up = down + np.uint32(0x10000)
    vd = down.view(np.float32).astype(np.float64)
    vu = up.view(np.float32).astype(np.float64)
    xv = x.astype(np.float64)
    dd = np.abs(xv - vd)
    du = np.abs(vu - xv)
    pick_up = (du < dd) | ((du == dd) & (((up >> np.uint32(16)) & np.uint32(1)) == 0))
    out = np.where(pick_up, up, down)
    return (out >> np.uint32(16)).astype(np.uint16)
