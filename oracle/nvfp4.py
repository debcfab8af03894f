"""Four Over Six (4/6) NVFP4 quantization and dequantization, step by step.

Method (Four Over Six documentation page, §Four Over Six): every NVFP4 block is
scaled adaptively so that its largest magnitude maps either to 6 or to 4, choosing
the one with the lower quantization error on the block's near-maximal values.
Format (Ultralytics glossary "FP4", §How FP4 works): 16 values share one FP8 E4M3
scale and the tensor has a second, FP32 scale; the classic rule maps the block
maximum to 6, the largest E2M1 magnitude.

Arithmetic, in the order executed (float32 IEEE, round-to-nearest-even, subnormals
kept; "RN(.)" is one fp32 rounding):

  O0  x = fp32 of the bf16 input (exact).  cols % 16 == 0; rows % 16 == 0 when the
      column-wise or 2D layout is used.
  O1  (option) random-sign Hadamard transform of each 1D block (``hadamard.py``);
      the fp32 result replaces x everywhere below.
  O2  A = max |x| over the tensor; per-tensor scale t = RN(A / 2688), 2688 = 448*6
      (largest E4M3 value times largest E2M1 value), stored in decode direction.
  O3  blocks: row-wise = 16 consecutive values of a row; column-wise = 16
      consecutive rows of one column (the quantization of X transposed, stored as the
      rows of a [cols, rows/2] array); 2D = a 16x16 tile.
  O4  a = max |x| over the block (the whole tile for 2D).
  O5  for each candidate c in (6, 4) (6 alone for the 6-only rule):
        u_c  = RN(1 / RN(t * c))                   once per tensor (inf when t == 0)
        r_c  = 0 if a == 0 else RN(a * u_c)        block scale, real units
        S_c  = E4M3 round-to-nearest-even of r_c, saturating to 448
        D_c  = value of S_c;  d_c = RN(D_c * t)    block decode scale
        if d_c is zero or subnormal the candidate encodes every value as a signed
        zero; otherwise inv_c = RN(1 / d_c) and v_i = RN(x_i * inv_c);
        m_i  = E2M1 round-to-nearest-even of |v_i| (saturating at 6), or the
               stochastic rounding of O9;
        e_i  = RN(E(m_i) * d_c - |x_i|)            one rounding of the exact error
        err_c: acc = 0; for i ascending acc = RN(e_i * e_i + acc) (fused
               multiply-add, one rounding per step);
               2D: one such accumulation per tile row, then the 16 row partials are
               summed pairwise ((p0+p1)+(p2+p3))+... with plain fp32 additions.
  O6  choose 4 iff err_4 < err_6 (ties, including 0 == 0, go to 6).
  O7  nibble q_i = (sign bit of x_i) << 3 | m_i; byte k of a block holds q_2k in the
      low and q_2k+1 in the high nibble; scale byte S of the chosen candidate; 2D
      writes the tile's byte into all 16 row-block slots of the tile.
  O8  dequantize: d = RN(D * t) per block, value = RN(E(q) * d), sign from bit 3;
      bf16 output = bf16 round-to-nearest-even of that fp32 value.
  O9  stochastic rounding: block b (flat index in the output's own layout) draws one
      Philox4x32-10 output with key = sr_seed, counter = (b_lo32, b_hi32, 0, stream)
      (stream 0 row-wise, 1 column-wise); element i takes byte i of the 16 output
      bytes (byte (i % 4) of word i // 4), call it k in 0..255.  For |v| >= 6 the code
      is 6.  Otherwise lo/hi are the grid values around |v|, p = (|v| - lo)/(hi - lo)
      (exact), p22 = p truncated to 22 fractional bits, and the value rounds up to hi
      iff (k + 0.5)/256 < p22.  Both candidates use the same draws and the choice
      compares the errors of the rounded values.
      2D tiles take the draws of the row-wise layout for every output.
      Full resolution ("sr_full"): element i of block b takes the whole 32-bit word
      i % 4 of Philox4x32-10(key = sr_seed, counter = (b_lo32, b_hi32, i // 4,
      stream)), four calls per block; with u = its top 22 bits (word >> 10), the
      value rounds up iff p22 * 2^22 + u >= 2^22, so it rounds up with probability
      p22 exactly (p truncated to 22 fractional bits), with no dead zone near the grid
      points.  Everything else as above.

The element-wise scale uses a per-block reciprocal and the per-block scale uses a
per-tensor reciprocal (u_c); the error is the exact dequantization error rounded
once and is accumulated with fused multiply-adds.  These are readings: the pages fix
none of these rounding steps.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .formats import (E2M1_GRID, bf16_bits_to_f32, e2m1_rne_code, e4m3_rne_sat,
                      e4m3_value)
from .fparith import fma32
from .hadamard import irht_blocks, rht_blocks, rht_signs
from .philox import philox4x32_10, split_seed

F32 = np.float32
SCALE_DENOM = F32(448.0 * 6.0)
MIN_NORMAL = F32(2.0 ** -126)


@dataclass
class Config:
    rule: str = "4/6"            # "4/6" or "6"
    rounding: str = "rne"        # "rne", "sr" (8-bit draws) or "sr_full" (22-bit draws)
    block: str = "1d"            # "1d" or "2d"
    rows_out: bool = True        # row-wise output
    cols_out: bool = False       # column-wise (transposed) output
    hadamard: bool = False
    hadamard_seed: int = 0
    sr_seed: int = 0


# ---------------------------------------------------------------------------- O2

def tensor_scale_from_amax(amax) -> np.float32:
    """t = RN(A / 2688)."""
    with np.errstate(divide="ignore", invalid="ignore"):
        return F32(F32(amax) / SCALE_DENOM)


# ---------------------------------------------------------------------------- O9

def sr_bytes(block_ids: np.ndarray, seed: int, stream: int) -> np.ndarray:
    """(n,) flat block indices -> (n, 16) uint8 random bytes of O9."""
    b = np.asarray(block_ids, dtype=np.uint64)
    ctr = np.stack([b & np.uint64(0xFFFFFFFF), b >> np.uint64(32),
                    np.zeros_like(b), np.full_like(b, stream)], axis=-1)
    words = philox4x32_10(ctr, split_seed(seed))              # (n, 4) uint32
    out = np.empty(words.shape[:-1] + (16,), dtype=np.uint8)
    for i in range(16):
        out[..., i] = (words[..., i // 4] >> np.uint32(8 * (i % 4))) & np.uint32(0xFF)
    return out


def sr_words(block_ids: np.ndarray, seed: int, stream: int) -> np.ndarray:
    """(n,) flat block indices -> (n, 16) uint32 draw words of the full-resolution
    mode of O9: element i takes word i % 4 of the call with counter word 2 = i // 4."""
    b = np.asarray(block_ids, dtype=np.uint64)
    out = np.empty(b.shape + (16,), dtype=np.uint32)
    for j in range(4):
        ctr = np.stack([b & np.uint64(0xFFFFFFFF), b >> np.uint64(32),
                        np.full_like(b, j), np.full_like(b, stream)], axis=-1)
        words = philox4x32_10(ctr, split_seed(seed))          # (n, 4) uint32
        out[..., 4 * j:4 * j + 4] = words
    return out


def _grid_position(magnitude: np.ndarray):
    """For |v| >= 0: the codes of the grid values lo <= |v| < hi (lo == hi == 6 at and
    above 6) and p = (|v| - lo) / (hi - lo), exact in fp64 (the steps are powers of
    two)."""
    m = np.asarray(magnitude, dtype=np.float64)
    lo = np.searchsorted(E2M1_GRID, m, side="right") - 1     # grid[lo] <= m
    lo = np.clip(lo, 0, 7)
    hi = np.minimum(lo + 1, 7)
    step = E2M1_GRID[hi] - E2M1_GRID[lo]
    p = np.where(step > 0, (m - E2M1_GRID[lo]) / np.where(step > 0, step, 1.0), 0.0)
    return lo, hi, p


def e2m1_sr_full_code(magnitude: np.ndarray, words: np.ndarray) -> np.ndarray:
    """Full-resolution stochastic rounding of |v| >= 0 onto the E2M1 grid with 32-bit
    draw words: with P = floor(p * 2^22) (p's first 22 fractional bits) and u = word >>
    10, |v| rounds up iff P + u >= 2^22.  Over the 2^22 values of u exactly P round up,
    so the chance is p to within 2^-22.  6 and above give 6."""
    lo, hi, p = _grid_position(magnitude)
    P = np.floor(p * 2.0 ** 22).astype(np.int64)
    u = (np.asarray(words, dtype=np.uint32) >> np.uint32(10)).astype(np.int64)
    up = (P + u) >= (1 << 22)
    code = np.where(up, hi, lo)
    code = np.where(np.asarray(magnitude, dtype=np.float64) >= 6.0, 7, code)
    return code.astype(np.uint8)


def e2m1_sr_code(magnitude: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Stochastic rounding of |v| >= 0 onto the E2M1 grid with draw k in 0..255.

    The position p of |v| between its grid neighbours is exact in fp64 (the grid steps
    are powers of two) and is truncated to 22 fractional bits before it is compared
    with the draw's threshold (k + 0.5)/256; the truncation moves the probability of
    rounding up by less than 2^-22."""
    m = np.asarray(magnitude, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    lo = np.searchsorted(E2M1_GRID, m, side="right") - 1     # grid[lo] <= m
    lo = np.clip(lo, 0, 7)
    hi = np.minimum(lo + 1, 7)
    step = E2M1_GRID[hi] - E2M1_GRID[lo]
    p = np.where(step > 0, (m - E2M1_GRID[lo]) / np.where(step > 0, step, 1.0), 0.0)
    p22 = np.floor(p * 2.0 ** 22) / 2.0 ** 22
    up = ((k + 0.5) / 256.0) < p22
    code = np.where(up, hi, lo)
    code = np.where(m >= 6.0, 7, code)
    return code.astype(np.uint8)


# ---------------------------------------------------------------------------- O4-O6

def _exact_error(emag: np.ndarray, d: F32, xmag: np.ndarray) -> np.ndarray:
    """e = RN32(E * d - |x|): E*d is exact in fp64 (<= 26 significant bits) and the
    difference is asserted exact in fp64 (TwoSum error term == 0), so one rounding
    to fp32 gives the correctly rounded error."""
    p = emag.astype(np.float64) * np.asarray(d, dtype=np.float64)
    q = xmag.astype(np.float64)
    s = p - q
    bb = s - p
    err = (p - (s - bb)) + (-q - bb)
    assert np.all(err == 0.0), "fp64 difference not exact"
    return s.astype(F32)


def _candidate(x: np.ndarray, a: np.ndarray, t: F32, c: float,
               draws: Optional[np.ndarray], two_d: bool):
    """One candidate for all blocks at once.
    x: (n, 16) fp32 for 1D or (n, 16, 16) for 2D; a: (n,) block amax.
    Returns scale bytes (n,), magnitude codes (same shape as x), errors (n,)."""
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        u = F32(F32(1.0) / F32(t * F32(c)))
        r = np.where(a == 0, F32(0.0), (a * u).astype(F32)).astype(F32)
    S = e4m3_rne_sat(r)
    D = e4m3_value(S).astype(F32)
    d = (D * t).astype(F32)
    ok = d >= MIN_NORMAL
    with np.errstate(divide="ignore"):
        inv = np.where(ok, F32(1.0) / np.where(ok, d, F32(1.0)), F32(0.0)).astype(F32)
    shape_b = (-1,) + (1,) * (x.ndim - 1)
    v = (x * inv.reshape(shape_b)).astype(F32)
    vmag = np.abs(v)
    if draws is None:
        m = e2m1_rne_code(vmag.reshape(-1)).reshape(x.shape)
    elif draws.dtype == np.uint32:                 # full-resolution draw words
        m = e2m1_sr_full_code(vmag.reshape(-1), draws.reshape(-1)).reshape(x.shape)
    else:                                          # 8-bit draw bytes
        m = e2m1_sr_code(vmag.reshape(-1), draws.reshape(-1)).reshape(x.shape)
    m = np.where(ok.reshape(shape_b), m, np.uint8(0)).astype(np.uint8)
    emag = E2M1_GRID[m]
    dd = np.broadcast_to(d.reshape(shape_b), x.shape)
    e = _exact_error(emag, dd, np.abs(x))
    if not two_d:
        acc = np.zeros(x.shape[0], dtype=F32)
        for i in range(16):
            acc = fma32(e[:, i], e[:, i], acc)
        return S, m, acc
    rows = np.zeros(x.shape[:2], dtype=F32)                 # (n, 16) row partials
    for j in range(16):
        rows = fma32(e[:, :, j], e[:, :, j], rows)
    level = rows
    with np.errstate(over="ignore"):                        # huge blocks: fp32 sums overflow to inf
        while level.shape[1] > 1:                           # pairwise over rows
            level = (level[:, 0::2] + level[:, 1::2]).astype(F32)
    return S, m, level[:, 0]


def quantize_blocks(x: np.ndarray, t: F32, rule: str = "4/6",
                    draws: Optional[np.ndarray] = None, two_d: bool = False):
    """Quantize independent blocks with the tensor scale t.
    x: (n, 16) or (n, 16, 16) fp32.  Returns (nibbles with sign, scale bytes,
    chose4 flags, err6, err4)."""
    x = np.asarray(x, dtype=F32)
    t = F32(t)
    axes = tuple(range(1, x.ndim))
    a = np.max(np.abs(x), axis=axes).astype(F32)
    S6, m6, e6 = _candidate(x, a, t, 6.0, draws, two_d)
    if rule == "4/6":
        S4, m4, e4 = _candidate(x, a, t, 4.0, draws, two_d)
        use4 = e4 < e6
    elif rule == "6":
        S4, m4, e4 = S6, m6, e6
        use4 = np.zeros(a.shape, dtype=bool)
    else:
        raise ValueError(rule)
    shape_b = (-1,) + (1,) * (x.ndim - 1)
    m = np.where(use4.reshape(shape_b), m4, m6)
    S = np.where(use4, S4, S6).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8)
    q = (sign << 3 | m).astype(np.uint8)
    return q, S, use4, e6, e4


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """(..., 2k) nibbles -> (..., k) bytes, element 2j in the low nibble."""
    q = np.asarray(q, dtype=np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


# ---------------------------------------------------------------------------- tensor

def prepare(x_bf16: np.ndarray, cfg: Config):
    """Return the fp32 values the blocks see (after the optional transform) in the
    orientation the transform uses, plus the tensor scale t (O0-O2)."""
    xb = np.asarray(x_bf16)
    if xb.dtype == np.uint16:
        x = bf16_bits_to_f32(xb)
    else:
        x = np.asarray(xb, dtype=F32)
    R, C = x.shape
    assert C % 16 == 0, "cols must be a multiple of 16"
    if cfg.cols_out or cfg.block == "2d":
        assert R % 16 == 0, "rows must be a multiple of 16"
    if cfg.hadamard:
        assert cfg.block == "1d" and (cfg.rows_out != cfg.cols_out)
        s = rht_signs(cfg.hadamard_seed)
        if cfg.rows_out:
            x = rht_blocks(x.reshape(R, C // 16, 16), s).reshape(R, C)
        else:
            xt = rht_blocks(x.T.reshape(C, R // 16, 16), s).reshape(C, R)
            x = np.ascontiguousarray(xt.T)
    amax = F32(np.max(np.abs(x))) if x.size else F32(0.0)
    return x, tensor_scale_from_amax(amax)


def quantize(x_bf16: np.ndarray, cfg: Config, t: Optional[F32] = None):
    """Full-tensor quantization.  x_bf16: (R, C) uint16 bf16 patterns (or fp32).
    Returns dict with 't', and 'row_data', 'row_scales', 'col_data', 'col_scales'
    for the requested outputs.  ``t`` overrides the tensor scale (for sampled
    checks of large tensors, where it is computed separately)."""
    x, t_own = prepare(x_bf16, cfg)
    t = t_own if t is None else F32(t)
    R, C = x.shape
    out = {"t": t}
    sr = cfg.rounding in ("sr", "sr_full")
    draw = sr_words if cfg.rounding == "sr_full" else sr_bytes
    if cfg.block == "2d":
        tiles = x.reshape(R // 16, 16, C // 16, 16).transpose(0, 2, 1, 3).reshape(-1, 16, 16)
        draws = None
        if sr:
            ids = np.arange(R * (C // 16), dtype=np.uint64)   # row-wise block ids
            draws = draw(ids, cfg.sr_seed, 0).reshape(R // 16, 16, C // 16, 16)
            draws = draws.transpose(0, 2, 1, 3).reshape(-1, 16, 16)
        q, S, _, _, _ = quantize_blocks(tiles, t, cfg.rule, draws, two_d=True)
        qf = q.reshape(R // 16, C // 16, 16, 16).transpose(0, 2, 1, 3).reshape(R, C)
        Sf = np.repeat(S.reshape(R // 16, C // 16), 16, axis=0)    # (R, C/16)
        if cfg.rows_out:
            out["row_data"] = pack_nibbles(qf)
            out["row_scales"] = Sf
        if cfg.cols_out:
            out["col_data"] = pack_nibbles(np.ascontiguousarray(qf.T))
            out["col_scales"] = np.repeat(S.reshape(R // 16, C // 16).T, 16, axis=0)
        return out
    if cfg.rows_out:
        blocks = x.reshape(-1, 16)
        draws = draw(np.arange(blocks.shape[0], dtype=np.uint64), cfg.sr_seed, 0) if sr else None
        q, S, _, _, _ = quantize_blocks(blocks, t, cfg.rule, draws)
        out["row_data"] = pack_nibbles(q).reshape(R, C // 2)
        out["row_scales"] = S.reshape(R, C // 16)
    if cfg.cols_out:
        blocks = np.ascontiguousarray(x.T).reshape(-1, 16)
        draws = draw(np.arange(blocks.shape[0], dtype=np.uint64), cfg.sr_seed, 1) if sr else None
        q, S, _, _, _ = quantize_blocks(blocks, t, cfg.rule, draws)
        out["col_data"] = pack_nibbles(q).reshape(C, R // 2)
        out["col_scales"] = S.reshape(C, R // 16)
    return out


def quantize_rows_sampled(x_bf16: np.ndarray, cfg: Config, t: F32, row_ids) -> dict:
    """Row-wise 1D output for the selected rows only, given the tensor scale t (for
    checks at full size: blocks are independent once t is known)."""
    assert cfg.block == "1d" and cfg.rows_out
    xb = np.asarray(x_bf16)
    R, C = xb.shape
    x = bf16_bits_to_f32(xb[row_ids]) if xb.dtype == np.uint16 else np.asarray(xb[row_ids], F32)
    if cfg.hadamard:
        x = rht_blocks(x.reshape(len(row_ids), C // 16, 16), rht_signs(cfg.hadamard_seed)).reshape(len(row_ids), C)
    blocks = x.reshape(-1, 16)
    draws = None
    if cfg.rounding in ("sr", "sr_full"):
        ids = (np.asarray(row_ids, dtype=np.uint64)[:, None] * np.uint64(C // 16)
               + np.arange(C // 16, dtype=np.uint64)[None, :]).reshape(-1)
        draws = (sr_words if cfg.rounding == "sr_full" else sr_bytes)(ids, cfg.sr_seed, 0)
    q, S, _, _, _ = quantize_blocks(blocks, F32(t), cfg.rule, draws)
    return {"row_data": pack_nibbles(q).reshape(len(row_ids), C // 2),
            "row_scales": S.reshape(len(row_ids), C // 16)}


def dequantize(data: np.ndarray, scales: np.ndarray, t) -> np.ndarray:
    """O8: data (R, C/2) bytes, scales (R, C/16) E4M3 bytes -> (R, C) fp32."""
    data = np.asarray(data, dtype=np.uint8)
    R = data.shape[0]
    C = data.shape[1] * 2
    q = unpack_nibbles(data).reshape(R, C // 16, 16)
    D = e4m3_value(np.asarray(scales, dtype=np.uint8)).astype(F32)
    d = (D * F32(t)).astype(F32)                                  # (R, C/16)
    mag = E2M1_GRID[q & 7]
    val = (mag * d[..., None].astype(np.float64)).astype(F32)      # one rounding
    val = np.where((q & 8) != 0, -val, val).astype(F32)
    return val.reshape(R, C)


def dequantize_hadamard(data: np.ndarray, scales: np.ndarray, t, seed: int) -> np.ndarray:
    """Dequantize a record made with the random Hadamard transform (seed ``seed``) and
    return it to the original basis: O8, then the inverse transform of every
    16-value block of the record's rows (fp32)."""
    val = dequantize(data, scales, t)
    R, C = val.shape
    back = irht_blocks(val.reshape(-1, 16), rht_signs(seed))
    return back.reshape(R, C).astype(F32)
