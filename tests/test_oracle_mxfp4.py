"""Pins for the oracle's MXFP4 path (CPU only).

Ultralytics glossary "FP4", §How FP4 works: MXFP4 puts 32 E2M1 values under one
power-of-two E8M0 scale (OCP Microscaling specification).  The scale rule is the OCP
specification's (floor(log2 amax) - 2); these tests pin it by closed forms, by the
properties the rule implies, and by exact rational arithmetic for the GEMM reference.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import mxfp4 as MX

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _one_block(vals):
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :len(vals)] = vals
    q = MX.quantize(x)
    codes = np.concatenate([q["data"][0] & 0xF, q["data"][0] >> 4]).reshape(2, 16).T.reshape(32)
    return int(q["scales"][0, 0]), codes, q


def test_closed_forms():
    # max 6 * 2^k: e = k, the max encodes as 6 (code 7)
    for k in (-10, 0, 3, 20):
        s, c, _ = _one_block([6.0 * 2.0 ** k, 1.0 * 2.0 ** k])
        assert s == 127 + k and c[0] == 7 and c[1] == 2
    # max 7: e = 0, 7 saturates to 6
    s, c, _ = _one_block([7.0, -7.5])
    assert s == 127 and c[0] == 7 and c[1] == 0xF
    # max 1: e = -2, so 1 -> 4 (code 6) and 0.3 -> 1.2 -> 1 (code 2)
    s, c, _ = _one_block([1.0, 0.3])
    assert s == 125 and c[0] == 6 and c[1] == 2
    # ties to even: with e = 0, 0.25 -> 0 (code 0), 0.75 -> 1 (code 2), 2.5 -> 2, 5 -> 4
    s, c, _ = _one_block([4.0, 0.25, 0.75, 2.5, 5.0])
    assert s == 127 and list(c[:5]) == [6, 0, 2, 4, 6]
    # zeros: e = -127 (byte 0); negative zero keeps its sign
    s, c, _ = _one_block([0.0, -0.0])
    assert s == 0 and c[0] == 0 and c[1] == 8


def test_scale_puts_the_block_max_in_4_to_8():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-30, 30, (64, 1)))).astype(np.float32)
    xb = F.f32_to_bf16_bits(x)
    xf = F.bf16_bits_to_f32(xb).reshape(64, 8, 32).astype(np.float64)
    q = MX.quantize(xb)
    e = q["scales"].astype(np.int64) - 127
    ratio = np.max(np.abs(xf), axis=-1) / np.exp2(e)
    assert np.all((ratio >= 4) & (ratio < 8))
    # every element's error: half a grid step where it is not saturated, else |v| - 6
    deq = MX.dequantize(q["data"], q["scales"]).reshape(64, 8, 32).astype(np.float64)
    v = np.abs(xf) / np.exp2(e)[..., None]
    step = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    bound = np.where(v > 6, v - 6, step / 2) * np.exp2(e)[..., None]
    assert np.all(np.abs(deq - xf) <= bound)


def test_brute_force_nearest_grid_value():
    """Each element code is the nearest signed grid value to V / 2^e (ties to even
    code), found by scanning all 16 codes."""
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((8, 64)) * 3).astype(np.float32)
    q = MX.quantize(x)
    e = q["scales"].astype(np.int64) - 127
    codes = np.zeros((8, 64), dtype=np.int64)
    codes[:, 0::2] = q["data"] & 0xF
    codes[:, 1::2] = q["data"] >> 4
    for r in range(8):
        for c in range(64):
            v = Fraction(float(x[r, c])) / Fraction(2) ** int(e[r, c // 32])
            best = None
            for code in range(16):
                mag = Fraction(GRID[code & 7])
                val = -mag if code & 8 else mag
                if (code & 8) != (1 if v < 0 or (v == 0 and np.signbit(x[r, c])) else 0) * 8:
                    continue
                d = abs(val - min(max(v, Fraction(-6)), Fraction(6)))
                key = (d, (code & 7) % 2)          # ties: even magnitude code
                if best is None or key < best[0]:
                    best = (key, code)
            assert codes[r, c] == best[1], (r, c, float(v))


def test_round_trip_of_representable_tensors():
    """Values that are grid points times the block's power of two come back exactly."""
    rng = np.random.default_rng(3)
    g = np.array(GRID)[rng.integers(0, 8, (16, 128))] * rng.choice([-1, 1], (16, 128))
    g.reshape(16, 4, 32)[:, :, 0] = 6.0                     # block max 6 -> e = k
    k = rng.integers(-20, 20, (16, 4))
    x = (g.reshape(16, 4, 32) * np.exp2(k)[..., None]).reshape(16, 128).astype(np.float32)
    q = MX.quantize(x)
    assert np.array_equal(MX.dequantize(q["data"], q["scales"]), x)


def test_gemm_reference_is_exact_rational_product():
    rng = np.random.default_rng(4)
    a = (rng.standard_normal((5, 64)) * 4).astype(np.float32)
    b = (rng.standard_normal((3, 64)) / 8).astype(np.float32)
    qa, qb = MX.quantize(a), MX.quantize(b)
    y = MX.gemm_ref64(qa["data"], qa["scales"], qb["data"], qb["scales"])
    da = MX.dequantize(qa["data"], qa["scales"])
    db = MX.dequantize(qb["data"], qb["scales"])
    for m in range(5):
        for n in range(3):
            exact = sum(Fraction(float(u)) * Fraction(float(v)) for u, v in zip(da[m], db[n]))
            assert abs(Fraction(y[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


@pytest.mark.parametrize("bad_cols", [16, 48])
def test_cols_must_be_whole_blocks(bad_cols):
    with pytest.raises(AssertionError):
        MX.quantize(np.zeros((2, bad_cols), dtype=np.float32))
