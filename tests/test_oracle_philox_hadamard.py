"""Pins for the oracle's Philox4x32-10 and random Hadamard transform (CPU only).

Philox: compared word for word with PyTorch's header-only Philox engine
(ATen/core/PhiloxRNGEngine.h), compiled here with g++; that engine maps
(seed, subsequence, offset) to key = seed and counter = (offset, subsequence).
Hadamard: compared with scipy.linalg.hadamard(16) (Sylvester order) in fp64.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle.hadamard import rht_blocks, rht_signs
from oracle.nvfp4 import sr_bytes, sr_words
from oracle.philox import philox4x32_10, split_seed

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def torch_philox():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    d = tempfile.mkdtemp()
    exe = os.path.join(d, "phx")
    subprocess.run([gxx, "-std=c++17", "-O1", "-I", inc,
                    os.path.join(HERE, "philox_torch_harness.cpp"), "-o", exe],
                   check=True, capture_output=True)

    def run(seed, sub, off):
        out = subprocess.run([exe, str(seed), str(sub), str(off)], check=True,
                             capture_output=True, text=True).stdout.split()
        return [int(w, 16) for w in out]
    yield run
    shutil.rmtree(d, ignore_errors=True)


CASES = [(0, 0, 0), (1234, 0, 0), (1234, 1 << 32, 5), (0xDEADBEEFCAFEF00D, 3, 1 << 40),
         (0xFFFFFFFFFFFFFFFF, (1 << 64) - 1, (1 << 64) - 1), (7, 1 << 32, 123456789)]


@pytest.mark.parametrize("seed,sub,off", CASES)
def test_philox_matches_torch_engine(torch_philox, seed, sub, off):
    ctr = np.array([off & 0xFFFFFFFF, off >> 32, sub & 0xFFFFFFFF, sub >> 32], dtype=np.uint64)
    ours = [int(w) for w in philox4x32_10(ctr, split_seed(seed))]
    assert ours == torch_philox(seed, sub, off)


def test_sr_bytes_layout_matches_counter_mapping(torch_philox):
    # block b of stream s uses counter (b_lo, b_hi, 0, s): torch's offset = b,
    # subsequence = s << 32; element i takes byte i%4 of word i//4.
    for b, s in [(0, 0), (5, 0), (77, 1), ((1 << 33) + 9, 1)]:
        words = torch_philox(1234, s << 32, b)
        got = sr_bytes(np.array([b], dtype=np.uint64), 1234, s)[0]
        want = [(words[i // 4] >> (8 * (i % 4))) & 0xFF for i in range(16)]
        assert list(got) == want


def test_sr_words_layout_matches_counter_mapping(torch_philox):
    # full-resolution draws: element i of block b (stream s) takes word i % 4 of the
    # call with counter (b_lo, b_hi, i // 4, s): torch's offset = b, subsequence =
    # (i // 4) + (s << 32)
    for b, s in [(0, 0), (9, 1), ((1 << 35) + 3, 0)]:
        got = sr_words(np.array([b], dtype=np.uint64), 4321, s)[0]
        want = []
        for j in range(4):
            want += torch_philox(4321, j + (s << 32), b)
        assert [int(w) for w in got] == want


def test_philox_bytes_uniform():
    byt = sr_bytes(np.arange(1 << 16, dtype=np.uint64), 99, 0).reshape(-1)
    counts = np.bincount(byt, minlength=256)
    exp = byt.size / 256
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 350          # 255 dof: p ~ 1e-4 threshold


def test_hadamard_matches_scipy():
    H = scipy.linalg.hadamard(16).astype(np.float64)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2000, 16)).astype(np.float32)
    for seed in (0, 1, 1234, 2 ** 63 + 5):
        s = rht_signs(seed)
        y = rht_blocks(x, s).astype(np.float64)
        ref = (0.25 * (H @ (s.astype(np.float64)[:, None] * x.astype(np.float64).T))).T
        err = np.abs(y - ref).max() / np.abs(ref).max()
        assert err < 4e-7
        # norm preserved (orthogonal transform)
        assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x.astype(np.float64), axis=1),
                           rtol=1e-6)


def test_hadamard_one_hot_is_signed_column():
    H = scipy.linalg.hadamard(16)
    s = rht_signs(1234)
    for k in range(16):
        e = np.zeros((1, 16), np.float32)
        e[0, k] = 1.0
        y = rht_blocks(e, s)[0]
        assert np.array_equal(y, (s[k] * 0.25 * H[:, k]).astype(np.float32))


def test_hadamard_round_trip():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((500, 16)).astype(np.float32)
    s = rht_signs(42)
    y = rht_blocks(x, s)
    back = rht_blocks(y, np.ones(16, np.float32)) * s        # (H/4)^-1 = H/4, then S^-1
    assert np.allclose(back, x, rtol=0, atol=1e-6 * np.abs(x).max())


def test_rht_signs_from_philox_word0():
    w0 = int(philox4x32_10(np.zeros(4, np.uint64), split_seed(0))[0])   # 0x6627e8d5
    assert w0 == 0x6627E8D5
    s = rht_signs(0)
    assert [int(v < 0) for v in s] == [(w0 >> k) & 1 for k in range(16)]


# ------------------------------------------------------------------ inverse transform

def test_inverse_hadamard_exact_round_trip_on_small_integers():
    """Small integer blocks: every fp32 operation of both transforms is exact (sums of
    at most 16 quarter-integers), so the round trip returns the input bit for bit."""
    from oracle.hadamard import irht_blocks
    rng = np.random.default_rng(3)
    x = rng.integers(-8, 9, size=(64, 16)).astype(np.float32)
    for seed in (0, 1, 99, 2 ** 40 + 7):
        s = rht_signs(seed)
        back = irht_blocks(rht_blocks(x, s), s)
        assert np.array_equal(back, x)


def test_inverse_hadamard_matches_scipy():
    """irht(y) = S (H/4) y in fp64, within fp32 rounding of the butterflies."""
    from oracle.hadamard import irht_blocks
    H = scipy.linalg.hadamard(16).astype(np.float64)
    rng = np.random.default_rng(4)
    y = rng.standard_normal((32, 16)).astype(np.float32)
    for seed in (5, 6):
        s = rht_signs(seed).astype(np.float64)
        want = (y.astype(np.float64) @ (H / 4.0).T) * s
        got = irht_blocks(y, rht_signs(seed)).astype(np.float64)
        assert np.max(np.abs(got - want)) <= 8 * 2.0 ** -24 * np.max(np.abs(y)) * 4


def test_dequantize_hadamard_returns_to_the_original_basis():
    """quantize with the transform, dequantize with the inverse: back to x within the
    format's error; the wrong seed gives garbage."""
    from oracle import formats as F
    from oracle import nvfp4 as N
    rng = np.random.default_rng(8)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    xb = F.f32_to_bf16_bits(x)
    xf = F.bf16_bits_to_f32(xb).astype(np.float64)
    for cfg in (N.Config(hadamard=True, hadamard_seed=21),
                N.Config(rows_out=False, cols_out=True, hadamard=True, hadamard_seed=21)):
        q = N.quantize(xb, cfg)
        lay = "row" if cfg.rows_out else "col"
        ref = xf if lay == "row" else xf.T
        good = N.dequantize_hadamard(q[f"{lay}_data"], q[f"{lay}_scales"], q["t"], 21)
        bad = N.dequantize_hadamard(q[f"{lay}_data"], q[f"{lay}_scales"], q["t"], 22)
        rel = lambda v: np.linalg.norm(v.astype(np.float64) - ref) / np.linalg.norm(ref)
        assert rel(good) < 0.15
        assert rel(bad) > 0.5
