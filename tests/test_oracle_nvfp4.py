"""Pins for the oracle's 4/6 NVFP4 quantize / dequantize (CPU only).

What pins it, besides itself:
  * the worked example on the Ultralytics glossary page "FP4" (§How FP4 works): the
    page's printed mean absolute errors (tests/golden), and the NVFP4 codec's errors
    on the same data must keep the page's ordering and magnitude;
  * closed-form blocks worked out by hand in fp32 (t = 1 exactly);
  * brute force over every E4M3 scale on tiny blocks;
  * the method's own claim (Four Over Six documentation page, §Four Over Six) that
    choosing between max->6 and max->4 never increases the block error;
  * metamorphic relations (sign, powers of two, permutations, transposition);
  * degenerate inputs.
"""
import json
import os

import numpy as np
import pytest
import torch

from fp4_block_quantization_amd import workloads as W
from oracle import formats as F
from oracle import nvfp4 as N
from oracle import page_example as PE

HERE = os.path.dirname(os.path.abspath(__file__))
F32 = np.float32


def bf16(x):
    return F.f32_to_bf16_bits(np.asarray(x, dtype=F32))


# ------------------------------------------------------------------ worked example

def test_page_worked_example_printed_errors():
    golden = json.load(open(os.path.join(HERE, "golden", "page_fp4_worked_example.json")))
    x = W.page_example().numpy()
    for block, want in golden["mae_printed"].items():
        got = PE.block_scale_mae(x, int(block))
        assert round(got, golden["decimals"]) == want, (block, got, want)


def test_nvfp4_codec_on_worked_example_keeps_ordering_and_magnitude():
    x = W.page_example().numpy()
    mae6, mse6 = PE.nvfp4_errors(x, "6")
    mae46, mse46 = PE.nvfp4_errors(x, "4/6")
    one_scale = PE.block_scale_mae(x, 4096)
    b32 = PE.block_scale_mae(x, 32)
    # 16-value blocks with E4M3 scales stay below the single-scale and 32-block errors
    for mae in (mae6, mae46):
        assert mae < b32 < one_scale
        assert abs(mae - 0.0747) / 0.0747 < 0.25      # page's 16-block magnitude
    assert mse46 <= mse6                             # 4/6 never increases squared error


def test_page_tie_rule_is_nearest_with_ties_to_the_smaller_magnitude():
    """The worked example's rounding: nearest grid point, first (smaller) one on an
    exact tie; checked by brute force over every midpoint and around it."""
    grid = F.E2M1_GRID
    mids = (grid[:-1] + grid[1:]) / 2
    assert np.array_equal(F.e2m1_nearest_lower_code(mids), np.arange(7))
    for m, i in zip(mids, range(7)):
        above = np.nextafter(m, np.inf)
        assert F.e2m1_nearest_lower_code(np.array([above]))[0] == i + 1
    rng = np.random.default_rng(12)
    v = np.concatenate([rng.uniform(0, 8, 20000), grid, [100.0]])
    want = np.array([int(np.argmin(np.abs(grid - a))) for a in v])   # first minimum
    assert np.array_equal(F.e2m1_nearest_lower_code(v), want)


# ------------------------------------------------------------------ closed forms

def _one_block_tensor(block_vals, extra_rows=1):
    """Tensor whose row 0 holds a 2688-block (so A = 2688 and t = 1 exactly) and
    whose row 1 holds the block under test."""
    x = np.zeros((1 + extra_rows, 16), F32)
    x[0, 0] = 2688.0
    x[1, :len(block_vals)] = block_vals
    return bf16(x)


def test_closed_form_six_and_four_point_five_picks_four():
    q = N.quantize(_one_block_tensor([6.0, 4.5]), N.Config())
    assert q["t"] == F32(1.0)
    # candidate 6: S=0x38 (1.0), 4.5 ties to 4 -> err 0.25; candidate 4: S=0x3C (1.5),
    # inv = RN(2/3): 6 -> 4.0 (code 6), 4.5 -> 3.0 (code 5), err 0 -> choose 4.
    assert q["row_scales"][1, 0] == 0x3C
    assert q["row_data"][1, 0] == (6 | 5 << 4)
    assert np.all(q["row_data"][1, 1:] == 0)
    # the 2688 block: r6 = 448 exactly and r4 = 672 saturates to 448 too -> tie -> 6
    assert q["row_scales"][0, 0] == 0x7E
    assert q["row_data"][0, 0] == 7


def test_closed_form_equal_values_pick_four():
    # 16 x 1.0: candidate 6 has S = 0x23 (0.171875) and every value -> 6*0.171875,
    # err = 16 * 2^-10; candidate 4 has S = 0x28 (0.25) and is exact.
    q = N.quantize(_one_block_tensor([1.0] * 16), N.Config())
    assert q["row_scales"][1, 0] == 0x28
    assert np.all(q["row_data"][1] == (6 | 6 << 4))
    q6 = N.quantize(_one_block_tensor([1.0] * 16), N.Config(rule="6"))
    assert q6["row_scales"][1, 0] == 0x23
    assert np.all(q6["row_data"][1] == (7 | 7 << 4))


def test_closed_form_exact_on_both_ties_to_six():
    # {6, 1}: candidate 6 (S = 1.0) is exact; candidate 4 (S = 1.5): 6 -> 4.0 exact,
    # 1 -> v = 2/3 -> 0.5 -> 0.75 (err 0.0625); candidate 6 wins.  {6}: both exact ->
    # tie -> 6.
    q = N.quantize(_one_block_tensor([6.0, 1.0]), N.Config())
    assert q["row_scales"][1, 0] == 0x38 and q["row_data"][1, 0] == (7 | 2 << 4)
    q = N.quantize(_one_block_tensor([6.0]), N.Config())
    assert q["row_scales"][1, 0] == 0x38 and q["row_data"][1, 0] == 7


def test_dequantize_closed_form():
    q = N.quantize(_one_block_tensor([6.0, 4.5, -1.0]), N.Config())
    y = N.dequantize(q["row_data"], q["row_scales"], q["t"])
    # candidate 4 wins (err 0.0625 vs 0.25): d = 1.5, and -1 -> v = -2/3 -> -0.5 -> -0.75
    assert y[1, 0] == 6.0 and y[1, 1] == 4.5 and y[1, 2] == -0.75 and y[0, 0] == 2688.0


# ------------------------------------------------------------------ brute force

def _exact_block_sse(x, d):
    """fp64 SSE of nearest-even rounding of x/d (exact real division)."""
    v = np.abs(x.astype(np.float64)) / d
    m = F.e2m1_rne_code(v)
    return float(np.sum((F.E2M1_GRID[m] * d - np.abs(x.astype(np.float64))) ** 2))


def test_brute_force_scale_search_tiny_blocks():
    rng = np.random.default_rng(7)
    n_ok = 0
    for trial in range(300):
        xb = bf16(np.concatenate([[2688.0 * rng.uniform(0.5, 1.0)],
                                  rng.standard_normal(15) * rng.uniform(0.1, 100)]))
        x = bf16(np.zeros((2, 16)))
        x[1] = xb
        x[0, 0] = bf16([2688.0])[0]                     # A = 2688, t = 1
        q = N.quantize(x, N.Config())
        xv = F.bf16_bits_to_f32(x[1])
        a = np.max(np.abs(xv.astype(np.float64)))
        s6 = F.e4m3_rne_sat(np.array([a / 6.0]))[0]
        s4 = F.e4m3_rne_sat(np.array([a / 4.0]))[0]
        sse = {int(s): _exact_block_sse(xv, F.E4M3_TABLE[s]) for s in range(1, 0x7F)}
        best = min(sse.values())
        chosen = int(q["row_scales"][1, 0])
        # the chosen scale is one of the two candidates ...
        assert chosen in (s6, s4)
        # ... and the one with the lower exact SSE (near-ties excepted)
        lo, hi = sorted([sse[int(s6)], sse[int(s4)]])
        if hi - lo > 1e-6 * max(hi, 1e-30):
            assert sse[chosen] == lo
            n_ok += 1
        # the exhaustive optimum is never worse than 4/6, which never beats it
        assert best <= sse[chosen] * (1 + 1e-9)
        assert sse[chosen] <= sse[int(s6)] * (1 + 1e-6) + 1e-30
    assert n_ok > 100


def test_per_element_codes_are_nearest_grid_points():
    rng = np.random.default_rng(8)
    x = bf16(rng.standard_normal((64, 64)))
    q = N.quantize(x, N.Config())
    y = N.dequantize(q["row_data"], q["row_scales"], q["t"]).astype(np.float64)
    xv = F.bf16_bits_to_f32(x).astype(np.float64)
    D = F.e4m3_value(q["row_scales"])
    d = np.repeat((D * np.float64(q["t"])).astype(F32).astype(np.float64), 16, axis=1)
    # every value's dequantized magnitude is a nearest grid point of |x|/d
    # (within the one-ulp effect of scaling by the rounded reciprocal)
    ratio = np.abs(xv) / d
    dist_chosen = np.abs(np.abs(y) / d - ratio)
    dist_best = np.min(np.abs(ratio[..., None] - F.E2M1_GRID), axis=-1)
    assert np.all(dist_chosen <= dist_best + 1e-6 * np.maximum(ratio, 1))


# ------------------------------------------------------------------ invariants

@pytest.mark.parametrize("name", ["c1"])
def test_four_over_six_never_worse_than_six_only(name):
    x = W.make(name).view(torch.int16).numpy().view(np.uint16)
    xv = F.bf16_bits_to_f32(x).astype(np.float64)
    _, t = N.prepare(x, N.Config())
    blocks = F.bf16_bits_to_f32(x).reshape(-1, 16)
    q, S, use4, e6, e4 = N.quantize_blocks(blocks, t, "4/6")
    assert np.all(np.minimum(e4, e6) <= e6)
    assert np.all(np.where(use4, e4, e6) == np.minimum(e4, e6))
    assert use4.any() and (~use4).any()
    q46 = N.quantize(x, N.Config())
    q6 = N.quantize(x, N.Config(rule="6"))
    sse46 = np.sum((N.dequantize(q46["row_data"], q46["row_scales"], q46["t"]) - xv) ** 2)
    sse6 = np.sum((N.dequantize(q6["row_data"], q6["row_scales"], q6["t"]) - xv) ** 2)
    assert sse46 <= sse6 * (1 + 1e-6)


def test_two_d_error_not_worse_than_six_only():
    rng = np.random.default_rng(9)
    x = bf16(rng.standard_normal((64, 96)) * 0.02)
    xv = F.bf16_bits_to_f32(x).astype(np.float64)
    q46 = N.quantize(x, N.Config(block="2d"))
    q6 = N.quantize(x, N.Config(block="2d", rule="6"))
    s46 = np.sum((N.dequantize(q46["row_data"], q46["row_scales"], q46["t"]) - xv) ** 2)
    s6 = np.sum((N.dequantize(q6["row_data"], q6["row_scales"], q6["t"]) - xv) ** 2)
    assert s46 <= s6 * (1 + 1e-6)
    # one scale per 16x16 tile, replicated to its 16 row-blocks
    sc = q46["row_scales"].reshape(4, 16, 6)
    assert np.all(sc == sc[:, :1, :])


# ------------------------------------------------------------------ metamorphic

def _rand(rows, cols, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * scale
    x.reshape(-1)[::97] *= 30
    return bf16(x)


@pytest.mark.parametrize("cfg", [N.Config(), N.Config(rounding="sr", sr_seed=3),
                                 N.Config(rounding="sr_full", sr_seed=3, cols_out=True),
                                 N.Config(block="2d", cols_out=True),
                                 N.Config(block="2d", rounding="sr_full", sr_seed=4),
                                 N.Config(hadamard=True, hadamard_seed=11)])
def test_negation_flips_sign_bits_only(cfg):
    x = _rand(48, 64, 1)
    neg = x ^ np.uint16(0x8000)
    a, b = N.quantize(x, cfg), N.quantize(neg, cfg)
    assert a["t"] == b["t"]
    for k in ("row_data", "col_data"):
        if k in a:
            assert np.array_equal(a[k] ^ np.uint8(0x88), b[k])
            assert np.array_equal(a[k.replace("data", "scales")], b[k.replace("data", "scales")])


@pytest.mark.parametrize("k", [-3, 1, 4])
def test_power_of_two_scaling(k):
    x = _rand(32, 64, 2)
    xs = bf16(F.bf16_bits_to_f32(x) * F32(2.0 ** k))
    a, b = N.quantize(x, N.Config()), N.quantize(xs, N.Config())
    assert b["t"] == F32(a["t"] * F32(2.0 ** k))
    assert np.array_equal(a["row_data"], b["row_data"])
    assert np.array_equal(a["row_scales"], b["row_scales"])


def test_row_permutation():
    x = _rand(64, 48, 3)
    perm = np.random.default_rng(4).permutation(64)
    a, b = N.quantize(x, N.Config()), N.quantize(x[perm], N.Config())
    assert np.array_equal(a["row_data"][perm], b["row_data"])
    assert np.array_equal(a["row_scales"][perm], b["row_scales"])


def test_colwise_is_rowwise_of_transpose():
    x = _rand(64, 80, 5)
    a = N.quantize(x, N.Config(rows_out=False, cols_out=True))
    b = N.quantize(np.ascontiguousarray(x.T), N.Config())
    assert a["t"] == b["t"]
    assert np.array_equal(a["col_data"], b["row_data"])
    assert np.array_equal(a["col_scales"], b["row_scales"])


def test_two_d_colwise_is_transposed_rowwise():
    x = _rand(48, 64, 6)
    for cfg in (N.Config(block="2d", cols_out=True),
                N.Config(block="2d", cols_out=True, rounding="sr", sr_seed=9)):
        q = N.quantize(x, cfg)
        rn = N.unpack_nibbles(q["row_data"])
        cn = N.unpack_nibbles(q["col_data"])
        assert np.array_equal(rn.T, cn)
        assert np.array_equal(np.repeat(q["row_scales"][::16], 1, axis=0).T.repeat(16, axis=0),
                              q["col_scales"])


def test_hadamard_option_rotates_before_quantizing():
    x = _rand(32, 64, 7)
    q = N.quantize(x, N.Config(hadamard=True, hadamard_seed=5))
    from oracle.hadamard import rht_blocks, rht_signs
    y = rht_blocks(F.bf16_bits_to_f32(x).reshape(-1, 16), rht_signs(5)).reshape(32, 64)
    assert q["t"] == N.tensor_scale_from_amax(np.max(np.abs(y)))
    q2 = N.quantize(y, N.Config())                 # quantizing the rotated fp32 values
    assert np.array_equal(q["row_data"], q2["row_data"])
    assert np.array_equal(q["row_scales"], q2["row_scales"])


# ------------------------------------------------------------------ sampled rows

SAMPLED_CFGS = [N.Config(), N.Config(rule="6"), N.Config(rounding="sr", sr_seed=1234),
                N.Config(hadamard=True, hadamard_seed=5),
                N.Config(hadamard=True, hadamard_seed=0, rounding="sr", sr_seed=2 ** 40 + 7),
                N.Config(rounding="sr_full", sr_seed=77)]


@pytest.mark.parametrize("cfg", SAMPLED_CFGS, ids=["rne", "six", "sr", "rht", "rht_sr", "sr_full"])
def test_sampled_rows_equal_whole_tensor_rows(cfg):
    """quantize_rows_sampled (the expectation of the full-size GPU checks) gives, on
    any row subset -- unsorted, with gaps, first and last row included -- the rows of
    the whole-tensor quantize under the same tensor scale."""
    x = _rand(1024, 1024, 21, scale=0.3)                 # 2 MiB of bf16
    _, t = N.prepare(x, cfg)
    whole = N.quantize(x, cfg, t=t)
    assert whole["t"] == t
    rng = np.random.default_rng(22)
    rows = np.concatenate([[1023, 0], rng.choice(np.arange(1, 1023), 61, replace=False)])
    assert not np.all(np.diff(rows) > 0)                 # not sorted
    got = N.quantize_rows_sampled(x, cfg, t, rows)
    assert np.array_equal(got["row_data"], whole["row_data"][rows])
    assert np.array_equal(got["row_scales"], whole["row_scales"][rows])


def test_sampled_rows_block_ids_past_two_to_the_32(monkeypatch):
    """Stochastic-rounding draws of row r, block j use the row-major flat block id
    r * (C / 16) + j (uint64).  With C = 256 (16 blocks per row) the ids of rows near
    2^28 pass 2^32; a tensor of 2^28 + 64 rows is emulated by one repeated row (zero
    row stride), and the ids handed to the draw generator are compared with Python's
    exact integers."""
    C = 256
    base = _rand(1, C, 23)
    R = (1 << 28) + 64
    x = np.lib.stride_tricks.as_strided(base, shape=(R, C), strides=(0, base.strides[1]))
    rows = np.array([(1 << 28) + 63, (1 << 28) - 1, 5, (1 << 28)], dtype=np.int64)
    seen = []
    real = N.sr_bytes

    def spy(ids, seed, stream):
        seen.append(np.array(ids, dtype=np.uint64))
        return real(ids, seed, stream)
    monkeypatch.setattr(N, "sr_bytes", spy)
    cfg = N.Config(rounding="sr", sr_seed=99)
    got = N.quantize_rows_sampled(x, cfg, F32(0.01), rows)
    want = np.array([int(r) * (C // 16) + j for r in rows for j in range(C // 16)], dtype=np.uint64)
    assert len(seen) == 1 and np.array_equal(seen[0], want)
    assert int(want.max()) >= 2 ** 32 and int(want.min()) < 2 ** 32
    # rows with the same values but different ids get different draws and codes
    assert not np.array_equal(got["row_data"][0], got["row_data"][1])
    # and a row's codes equal those of the same values quantized as blocks with those ids
    blocks = F.bf16_bits_to_f32(base).reshape(-1, 16)
    q, S, _, _, _ = N.quantize_blocks(blocks, F32(0.01), "4/6", real(want[:16], 99, 0))
    assert np.array_equal(got["row_data"][0], N.pack_nibbles(q).reshape(-1))
    assert np.array_equal(got["row_scales"][0], S)


# ------------------------------------------------------------------ stochastic rounding

def test_sr_keeps_grid_values_and_is_unbiased():
    grid = F.E2M1_GRID
    for g in grid:
        codes = N.e2m1_sr_code(np.full(256, g), np.arange(256))
        assert np.all(grid[codes] == g)
    rng = np.random.default_rng(10)
    vals = rng.uniform(0, 6, 2000)
    for v in vals:
        codes = N.e2m1_sr_code(np.full(256, v), np.arange(256))
        out = grid[codes]
        lo = grid[grid <= v].max()
        hi = grid[grid > v].min() if v < 6 else 6.0
        assert set(np.unique(out)) <= {lo, hi}
        # exhaustive over the 256 draws: mean within 1/512 (the draws' resolution) plus
        # 2^-22 (the position's truncation) of a grid step of v
        assert abs(out.mean() - v) <= (hi - lo) * (1 / 512 + 2.0 ** -22) + 1e-12
    assert np.all(grid[N.e2m1_sr_code(np.array([6.0, 7.0, 100.0]), np.array([0, 128, 255]))] == 6)


def test_sr_position_is_truncated_to_22_fraction_bits():
    """Worked by hand: on [0.5, 1) the grid step is 0.5, so p = 2 (|v| - 0.5), and draw
    k = 0 has threshold q = 0.5/256 = 2^-9.  |v| = 0.5 + 2^-10 gives p = q exactly (no
    rounding up: the comparison is strict); one fp32 ulp (2^-24) above it p exceeds q by
    2^-23, which the truncation to 22 fractional bits drops (down); two ulps above, by
    2^-22, which it keeps (up).  Below 0.5 (step 0.5, lo = 0) the same holds at
    |v| = 2^-10 + 2^-30 (down) and 2^-10 + 2^-23 (up).  On [2, 4) (step 1, exact p) the
    threshold of k = 255 is 1 - 2^-9: |v| = 3 - 2^-9 stays at 2, the next fp32 value up
    rounds to 3."""
    grid = F.E2M1_GRID
    def up(v, k):
        c = N.e2m1_sr_code(np.array([np.float32(v)], dtype=np.float64), np.array([k]))[0]
        return grid[c] > v
    assert not up(0.5 + 2.0 ** -10, 0)
    assert not up(0.5 + 2.0 ** -10 + 2.0 ** -24, 0)
    assert up(0.5 + 2.0 ** -10 + 2.0 ** -23, 0)
    assert not up(2.0 ** -10 + 2.0 ** -30, 0)
    assert up(2.0 ** -10 + 2.0 ** -23, 0)
    assert not up(3.0 - 2.0 ** -9, 255)
    assert up(float(np.nextafter(np.float32(3.0 - 2.0 ** -9), np.float32(4.0))), 255)


def test_sr_draw_resolution_edges():
    """With one 8-bit draw per element the chance of rounding up is the number of draw
    bytes k with (k + 0.5) / 256 < p22, over 256.  Positions below 1/512 (and exactly
    1/512: the comparison is strict) never round up; positions above 511/512 always
    do; elsewhere the chance is within 2^-9 of p (plus the 2^-22 truncation), and the
    bias 2^-9 is reached at p = 1/512.  Checked exhaustively over the 256 draws on the
    step [2, 3), where p = |v| - 2 is exact in fp32."""
    k = np.arange(256)
    grid = F.E2M1_GRID

    def chance(p):
        v = np.float32(2.0 + p)
        assert np.float64(v) - 2.0 == p
        codes = N.e2m1_sr_code(np.full(256, np.float64(v)), k)
        return np.mean(grid[codes] > 2.0)
    for p in (2.0 ** -20, 2.0 ** -10, 1 / 512 - 2.0 ** -20, 1 / 512):
        assert chance(p) == 0.0, p
    assert chance(1 / 512 + 2.0 ** -20) == 1 / 256
    for p in (511 / 512 + 2.0 ** -20, 1 - 2.0 ** -21):
        assert chance(p) == 1.0, p
    assert chance(511 / 512) == 255 / 256
    rng = np.random.default_rng(13)
    ps = np.concatenate([rng.uniform(0, 1, 400), np.arange(1, 512) / 512])
    ps = np.floor(ps * 2.0 ** 21) / 2.0 ** 21            # exact in fp32 on [2, 3)
    bias = np.array([abs(chance(p) - p) for p in ps])
    assert bias.max() <= 2.0 ** -9
    assert abs(chance(1 / 512) - 1 / 512) == 2.0 ** -9


def _sr_full_chance(v):
    """Fraction of the 2^22 draw values u (low 10 bits of the word set to a fixed
    pattern, which the rule ignores) for which |v| rounds up under the full-resolution
    rule, and the up / down values."""
    u = np.arange(1 << 22, dtype=np.uint32)
    words = (u << np.uint32(10)) | np.uint32(0x2A5)
    codes = N.e2m1_sr_full_code(np.full(u.shape, v, dtype=np.float64), words)
    vals = F.E2M1_GRID[codes]
    return np.count_nonzero(vals > v) / float(1 << 22), np.unique(vals)


def test_sr_full_rounds_up_with_chance_p22():
    """Full-resolution stochastic rounding: over all 2^22 draw values exactly
    floor(p * 2^22) round up, so the chance is p when p has at most 22 fractional bits
    (every value at or above 1, e.g. on [2, 3) where p = |v| - 2) and p truncated to
    22 bits below 1.  No dead zone: p = 2^-22 rounds up for exactly one draw value,
    p = 1 - 2^-22 for all but one."""
    for p in (2.0 ** -22, 2.0 ** -21, 1 / 1024, 1 / 512, 0.3 - 0.3 % 2.0 ** -21,
              511 / 512 + 2.0 ** -20, 1 - 2.0 ** -22):
        v = 2.0 + p
        assert np.float64(np.float32(v)) == v
        chance, vals = _sr_full_chance(v)
        assert chance == p, (p, chance)
        assert set(vals) <= {2.0, 3.0}
    # below 1 the position has more than 22 bits: the chance is p truncated
    v = float(np.float32(0.5 + 2.0 ** -10 + 2.0 ** -24))        # p = 2^-9 + 2^-23
    chance, _ = _sr_full_chance(v)
    assert chance == 2.0 ** -9
    # grid values never move; 6 and above give 6
    for g in F.E2M1_GRID:
        chance, vals = _sr_full_chance(g)
        assert chance == 0.0 and list(vals) == [g]
    codes = N.e2m1_sr_full_code(np.array([6.0, 7.5, 1e30]), np.array([0, 2 ** 32 - 1, 12345], dtype=np.uint32))
    assert np.all(F.E2M1_GRID[codes] == 6.0)


def test_sr_full_has_no_dead_zone_where_8_bit_draws_have_one():
    """A value 1/1024 of a grid step above a grid point: the 8-bit draws never round it
    up (bias -1/1024 step), the full-resolution draws round it up for 1/1024 of the
    draws (no bias)."""
    v = 2.0 + 1 / 1024
    k = np.arange(256)
    assert np.all(F.E2M1_GRID[N.e2m1_sr_code(np.full(256, v), k)] == 2.0)
    chance, _ = _sr_full_chance(v)
    assert chance == 1 / 1024


def test_sr_full_tensor_is_unbiased_where_8_bit_is_not():
    """Quantizing a tensor whose values sit 1/1024 of a grid step above grid points:
    with 8-bit draws the dequantized mean stays on the grid points (biased low); with
    full-resolution draws it moves up by about 1/1024 of a step."""
    t = F32(1.0)
    # block {6, 2 + 1/1024 x 15} at t = 1: candidate 6 has d = 1 exactly (S = 1.0)
    blocks = np.full((4096, 16), 2.0 + 1 / 1024, dtype=F32)
    blocks[:, 0] = 6.0
    ids = np.arange(4096, dtype=np.uint64)
    q8, _, _, _, _ = N.quantize_blocks(blocks, t, "6", N.sr_bytes(ids, 5, 0))
    qf, _, _, _, _ = N.quantize_blocks(blocks, t, "6", N.sr_words(ids, 5, 0))
    v8 = F.E2M1_GRID[q8[:, 1:] & 7]
    vf = F.E2M1_GRID[qf[:, 1:] & 7]
    assert np.all(v8 == 2.0)
    n = vf.size
    ups = np.count_nonzero(vf == 3.0)
    assert np.all((vf == 2.0) | (vf == 3.0))
    # 61440 draws at chance 1/1024: mean 60, sd ~7.7
    assert abs(ups - n / 1024) < 5 * np.sqrt(n / 1024)


def test_sr_tensor_mean_close_to_input():
    x = _rand(64, 256, 11, scale=0.01)
    xv = F.bf16_bits_to_f32(x).astype(np.float64)
    q = N.quantize(x, N.Config(rounding="sr", sr_seed=1234))
    y = N.dequantize(q["row_data"], q["row_scales"], q["t"]).astype(np.float64)
    rne = N.quantize(x, N.Config())
    yr = N.dequantize(rne["row_data"], rne["row_scales"], rne["t"]).astype(np.float64)
    # SR error is unbiased: its mean is far smaller than its spread
    assert abs(np.mean(y - xv)) < 0.05 * np.std(y - xv)
    assert np.sum((yr - xv) ** 2) < np.sum((y - xv) ** 2)       # RNE has lower MSE


# ------------------------------------------------------------------ degenerate

def test_zero_tensor():
    x = bf16(np.zeros((32, 32)))
    x[3, 5] = np.uint16(0x8000)                                    # one -0.0
    q = N.quantize(x, N.Config(cols_out=True))
    assert q["t"] == 0.0
    assert np.all(q["row_scales"] == 0) and np.all(q["col_scales"] == 0)
    nib = N.unpack_nibbles(q["row_data"])
    assert nib[3, 5] == 8 and np.sum(nib) == 8
    y = N.dequantize(q["row_data"], q["row_scales"], q["t"])
    assert np.all(y == 0) and np.signbit(y[3, 5])


def test_single_nonzero_element():
    x = bf16(np.zeros((16, 32)))
    x[7, 20] = bf16([-3.25])[0]
    q = N.quantize(x, N.Config())
    y = N.dequantize(q["row_data"], q["row_scales"], q["t"])
    assert y[7, 20] == F32(-3.25)                                  # maps exactly to 6 * d
    assert np.count_nonzero(y) == 1


def test_tiny_tensor_underflow_is_consistent():
    # values in the bf16 subnormal range: the decode scale underflows, the block
    # encodes to signed zeros (or keeps a few codes) -- dequantize agrees with codes
    x = bf16(np.array([[1e-39, -3e-39, 2e-40, 0.0] * 4]))
    q = N.quantize(x, N.Config())
    y = N.dequantize(q["row_data"], q["row_scales"], q["t"])
    assert np.all(np.isfinite(y))
