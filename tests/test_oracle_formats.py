"""Pins for the oracle's number formats (CPU only).

E2M1: the value set printed on the Ultralytics glossary page "FP4" (opening section)
and round-to-nearest-even written as a threshold table (midpoints of the grid, ties to
the even code) -- an independent formulation of the oracle's brute-force nearest.
E4M3 and bfloat16: checked against PyTorch's own conversions (library routines).
"""
import numpy as np
import pytest
import torch

from oracle import formats as F


def test_e2m1_grid_matches_page_value_set():
    # page: 0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6
    assert list(F.E2M1_GRID) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    vals = F.e2m1_value(np.arange(16))
    assert sorted(set(np.abs(vals))) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.signbit(vals[8]) and vals[8] == 0.0          # code 8 is -0
    assert np.all(vals[9:] == -vals[1:8])


def _threshold_rule(m):
    """RNE onto {0,.5,1,1.5,2,3,4,6} as a threshold table; at a midpoint the even
    code wins: 0.25->0, 0.75->2 (1.0), 1.25->2, 1.75->4 (2.0), 2.5->4, 3.5->6 (4.0),
    5.0->6 (4.0); above 5 -> 7 (6.0, saturating)."""
    m = np.asarray(m, dtype=np.float64)
    code = np.zeros(m.shape, dtype=np.int64)
    code = np.where(m > 0.25, 1, code)
    code = np.where(m >= 0.75, 2, code)
    code = np.where(m > 1.25, 3, code)
    code = np.where(m >= 1.75, 4, code)
    code = np.where(m > 2.5, 5, code)
    code = np.where(m >= 3.5, 6, code)
    code = np.where(m > 5.0, 7, code)
    return code


def _fp32_near(values, ulps):
    out = []
    for v in values:
        b = np.array([v], dtype=np.float32).view(np.uint32)[0]
        lo = max(int(b) - ulps, 0)
        out.append(np.arange(lo, int(b) + ulps + 1, dtype=np.uint32).view(np.float32))
    return np.concatenate(out)


def test_e2m1_rne_matches_threshold_table():
    bf16 = np.arange(0, 0x7F80, dtype=np.uint16)            # every finite positive bf16
    pts = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 8.0, 0.5, 1.0, 2.0, 4.0]
    near = _fp32_near(pts, 4096)
    tiny = np.arange(0, 1 << 16, dtype=np.uint32).view(np.float32)   # zero + subnormals
    rng = np.random.default_rng(1)
    rnd = (rng.random(1 << 20) * 12).astype(np.float32)
    big = np.array([1e3, 1e10, 3.0e38, np.finfo(np.float32).max], dtype=np.float32)
    m = np.concatenate([F.bf16_bits_to_f32(bf16), near, tiny, rnd, big])
    assert np.array_equal(F.e2m1_rne_code(m).astype(np.int64), _threshold_rule(m))


def test_e4m3_table_matches_torch_decode():
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(F.E4M3_TABLE, tv)
    assert F.E4M3_TABLE[0x7E] == 448.0 and F.E4M3_TABLE[1] == 2.0 ** -9


def test_e4m3_rne_matches_torch_up_to_464():
    table = F.E4M3_TABLE
    mids = (table[:-1] + table[1:]) / 2
    near = _fp32_near(list(mids) + list(table[1:]), 64)
    bf16 = F.bf16_bits_to_f32(np.arange(0, 0x43E8, dtype=np.uint16))   # bf16 <= 464
    rng = np.random.default_rng(2)
    logu = np.exp(rng.uniform(np.log(2.0 ** -14), np.log(464.0), 1 << 20)).astype(np.float32)
    r = np.concatenate([near, bf16, logu, np.array([0.0, 2.0 ** -10, 3 * 2.0 ** -11], np.float32)])
    r = r[(r >= 0) & (r <= 464.0)]
    ours = F.e4m3_rne_sat(r)
    ref = torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # specific values: 2^-10 is a tie between 0 and 2^-9 -> 0 (even); 3*2^-11 -> 2^-9
    assert F.e4m3_rne_sat(np.array([2.0 ** -10]))[0] == 0
    assert F.e4m3_rne_sat(np.array([3 * 2.0 ** -11]))[0] == 1


def test_e4m3_saturates_above_448():
    r = np.array([448.0, 449.0, 464.0, 464.0001, 480.0, 1e6, np.inf, 3e38])
    assert np.all(F.e4m3_rne_sat(r) == 0x7E)


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(1 << 20).astype(np.float32) * np.float32(3.0)
    ties = ((rng.integers(0, 1 << 15, 4096, dtype=np.uint32) << 16)
            | np.uint32(0x8000)).view(np.float32)
    ties = ties[np.isfinite(ties)]
    x = np.concatenate([x, ties, np.array([0.0, -0.0, 1e-40, -1e-40], np.float32)])
    ours = F.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_roundtrip_exact():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    assert np.array_equal(F.f32_to_bf16_bits(F.bf16_bits_to_f32(bits)), bits)
