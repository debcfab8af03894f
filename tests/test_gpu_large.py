"""GPU parity past the 32-bit element index: a bf16 tensor of 131088 x 16400 =
2,149,843,200 elements (> 2^31, 4.3 GB) through every kernel family, checked against
the oracle on sampled rows, columns and tile rows (blocks are independent once the
tensor scale is known), including the row that straddles element 2^31 and the last
row.  16400 % 64 != 0, so the column-wise tiles have a ragged edge too.

Inputs are seeded: torch's generator on the device for the bf16 tensor and for the
random records the dequantize checks read.  The oracle sees the same values (copied
to the host), and its tensor scale comes from the host copy, never from the library.
"""
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import mxfp4 as MX
from oracle import nvfp4 as N

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
R, C = 131088, 16400
EDGE = (1 << 31) // C                    # row holding elements 2^31 - 2048 .. 2^31 + 14351


@pytest.fixture(scope="module")
def fos():
    from fp4_block_quantization_amd import fos as mod
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return mod


@pytest.fixture(scope="module")
def big():
    """(device bf16 tensor, host bf16 bit patterns, oracle tensor scale)."""
    assert R * C > (1 << 31) and EDGE * C < (1 << 31) < (EDGE + 1) * C
    g = torch.Generator(device=DEV)
    g.manual_seed(20240611)
    x = torch.randn(R, C, generator=g, device=DEV, dtype=torch.float32)
    # per-row powers of two, so block scales cover many E4M3 codes
    x *= torch.exp2(torch.randint(-6, 7, (R, 1), generator=g, device=DEV).float())
    x = x.to(torch.bfloat16)
    torch.cuda.synchronize()
    bits = x.view(torch.int16).cpu().numpy().view(np.uint16)
    # finite bf16 magnitudes order like their 15-bit patterns
    amax_bits = np.uint16(np.max(bits & np.uint16(0x7FFF)))
    t = N.tensor_scale_from_amax(F.bf16_bits_to_f32(np.array([amax_bits]))[0])
    yield x, bits, t
    del x
    torch.cuda.empty_cache()


def _rows(n, seed, limit=R, edge=EDGE):
    """n random row ids below `limit`, plus the first and last rows and (for a
    tensor's rows) the rows around the one holding element 2^31."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, edge - 1, edge, edge + 1, limit - 1] if edge else [0, limit - 1]
    return np.unique(np.concatenate([fixed, rng.choice(limit, n, replace=False)]))


def _host_rows(t: torch.Tensor, rows) -> np.ndarray:
    return t[torch.from_numpy(rows).to(DEV)].cpu().numpy()


def _same(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first {bad[:4].tolist()}"


def _t_bits(q):
    return np.float32(q.tensor_scale.cpu().numpy()[0]).view(np.uint32)


def test_row_wise_past_2_31(fos, big):
    x, bits, t = big
    q = fos.quantize(x)
    assert _t_bits(q) == t.view(np.uint32)
    rows = _rows(24, 1)
    o = N.quantize_rows_sampled(bits, N.Config(), t, rows)
    _same(_host_rows(q.data, rows), o["row_data"], "row_data")
    _same(_host_rows(q.scales, rows), o["row_scales"], "row_scales")


def test_row_and_column_wise_past_2_31(fos, big):
    x, bits, t = big
    qr, qc = fos.quantize(x, outputs=("row", "col"))
    assert _t_bits(qr) == t.view(np.uint32)
    rows = _rows(16, 2)
    o = N.quantize_rows_sampled(bits, N.Config(), t, rows)
    _same(_host_rows(qr.data, rows), o["row_data"], "row_data")
    _same(_host_rows(qr.scales, rows), o["row_scales"], "row_scales")
    cols = _rows(16, 3, limit=C, edge=None)
    cols = np.unique(np.concatenate([cols, [C - 17, C - 16]]))   # the ragged last tile
    xt = np.ascontiguousarray(bits[:, cols].T)
    oc = N.quantize_rows_sampled(xt, N.Config(), t, np.arange(len(cols)))
    _same(_host_rows(qc.data, cols), oc["row_data"], "col_data")
    _same(_host_rows(qc.scales, cols), oc["row_scales"], "col_scales")


def test_2d_past_2_31(fos, big):
    x, bits, t = big
    cfg = N.Config(block="2d")
    q = fos.quantize(x, block="2d")
    assert _t_bits(q) == t.view(np.uint32)
    for I in _rows(8, 4, limit=R // 16, edge=None).tolist() + [EDGE // 16]:
        o = N.quantize(bits[16 * I:16 * I + 16], cfg, t=t)
        sl = np.arange(16 * I, 16 * I + 16)
        _same(_host_rows(q.data, sl), o["row_data"], f"tile-row {I} data")
        _same(_host_rows(q.scales, sl), o["row_scales"], f"tile-row {I} scales")


def test_hadamard_sr_given_scale_past_2_31(fos, big):
    """Transform + stochastic rounding (Philox counters are global block ids) with
    the tensor scale given by the caller."""
    x, bits, t = big
    cfg = N.Config(hadamard=True, hadamard_seed=3, rounding="sr", sr_seed=(1 << 33) + 5)
    td = torch.tensor([t], dtype=torch.float32, device=DEV)
    q = fos.quantize(x, rounding="sr", sr_seed=cfg.sr_seed, hadamard_seed=3, tensor_scale=td)
    rows = _rows(12, 5)
    o = N.quantize_rows_sampled(bits, cfg, t, rows)
    _same(_host_rows(q.data, rows), o["row_data"], "row_data")
    _same(_host_rows(q.scales, rows), o["row_scales"], "row_scales")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dequantize_past_2_31(fos, big, dtype):
    """A random record (any nibble, finite non-negative E4M3 scale bytes) of the same
    shape; the oracle decodes the sampled rows."""
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    data = torch.randint(0, 256, (R, C // 2), generator=g, device=DEV, dtype=torch.uint8)
    scales = torch.randint(0, 127, (R, C // 16), generator=g, device=DEV, dtype=torch.uint8)
    t = np.float32(0.0123)
    rec = fos.NVFP4Tensor(data, scales, torch.tensor([t], dtype=torch.float32, device=DEV))
    y = fos.dequantize(rec, dtype)
    rows = _rows(12, 6)
    want = N.dequantize(_host_rows(data, rows), _host_rows(scales, rows), t)
    got = _host_rows(y.view(torch.int32 if dtype == torch.float32 else torch.int16), rows)
    if dtype == torch.float32:
        _same(got.view(np.uint32), want.view(np.uint32), "deq f32")
    else:
        _same(got.view(np.uint16), F.f32_to_bf16_bits(want), "deq bf16")
    del y, data, scales


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dequantize_hadamard_past_2_31(fos, big, dtype):
    """Inverse-Hadamard dequantize of a random record of the same shape: the kernel's
    workgroups loop over many 256-block ranges; sampled rows against the oracle."""
    g = torch.Generator(device=DEV)
    g.manual_seed(78)
    data = torch.randint(0, 256, (R, C // 2), generator=g, device=DEV, dtype=torch.uint8)
    scales = torch.randint(0, 127, (R, C // 16), generator=g, device=DEV, dtype=torch.uint8)
    t = np.float32(0.0071)
    rec = fos.NVFP4Tensor(data, scales, torch.tensor([t], dtype=torch.float32, device=DEV),
                          hadamard_seed=11)
    y = fos.dequantize(rec, dtype, inverse_hadamard=True)
    rows = _rows(12, 8)
    want = N.dequantize_hadamard(_host_rows(data, rows), _host_rows(scales, rows), t, 11)
    got = _host_rows(y.view(torch.int32 if dtype == torch.float32 else torch.int16), rows)
    if dtype == torch.float32:
        _same(got.view(np.uint32), want.view(np.uint32), "deq-rht f32")
    else:
        _same(got.view(np.uint16), F.f32_to_bf16_bits(want), "deq-rht bf16")
    del y, data, scales


def test_mxfp4_past_2_31(fos, big):
    """The same elements as a [65544, 32800] tensor (MXFP4 rows are whole 32-blocks)."""
    x, bits, _ = big
    r2, c2 = R // 2, 2 * C
    q = fos.mx_quantize(x.view(r2, c2))
    rows = _rows(16, 7, limit=r2, edge=(1 << 31) // c2)
    o = MX.quantize(bits.reshape(r2, c2)[rows])
    _same(_host_rows(q.data, rows), o["data"], "mx data")
    _same(_host_rows(q.scales, rows), o["scales"], "mx scales")
    y = fos.mx_dequantize(q, torch.float32)
    want = MX.dequantize(o["data"], o["scales"])
    _same(_host_rows(y.view(torch.int32), rows).view(np.uint32), want.view(np.uint32), "mx deq")
