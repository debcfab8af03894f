"""fos_quantize_noalloc (no workspace, the library's per-GPU scratch array) against
fos_quantize (caller's workspace), through the C ABI: bit-exact records and tensor
scale, on two calls in a row with the second input smaller, for every option that
changes the tensor-scale pass (plain, Hadamard along rows, Hadamard along columns)
and the layouts (row-wise, row + column-wise, 2D)."""
import ctypes

import numpy as np
import pytest
import torch

from fp4_block_quantization_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def fos():
    from fp4_block_quantization_amd import fos as mod
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return mod


def _outputs(R, C, outs):
    u8 = dict(dtype=torch.uint8, device=DEV)
    rd = rs = cd = cs = None
    if "row" in outs:
        rd, rs = torch.full((R, C // 2), 0xAB, **u8), torch.full((R, C // 16), 0xAB, **u8)
    if "col" in outs:
        cd, cs = torch.full((C, R // 2), 0xCD, **u8), torch.full((C, R // 16), 0xCD, **u8)
    return rd, rs, cd, cs, torch.full((1,), -1.0, dtype=torch.float32, device=DEV)


CASES = {
    "row_rne": dict(kw={}, outs=("row",)),
    "row_sr": dict(kw=dict(rounding="sr", sr_seed=1234), outs=("row",)),
    "rowcol": dict(kw=dict(outputs=("row", "col")), outs=("row", "col")),
    "row_rht_sr": dict(kw=dict(hadamard_seed=0, rounding="sr", sr_seed=7), outs=("row",)),
    "col_rht": dict(kw=dict(outputs=("col",), hadamard_seed=3), outs=("col",)),
    "2d": dict(kw=dict(block="2d"), outs=("row",)),
}
# first call large (the scale pass writes hundreds of partial maxima), second small
SHAPES = [(2048, 4096), (96, 160)]


@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_matches_quantize(fos, case):
    kw, outs = CASES[case]["kw"], CASES[case]["outs"]
    cfg = fos.make_config(**kw)
    for i, (R, C) in enumerate(SHAPES):
        print(f"noalloc {case} call {i}: {R}x{C}", flush=True)
        x = W.random_bf16(R, C, 31 + i, "student_t", scale=0.1 * (i + 1)).to(DEV)
        ref = _outputs(R, C, outs)
        got = _outputs(R, C, outs)
        fos.fos_quantize(cfg, x, *ref[:4], ref[4])
        fos.fos_quantize_noalloc(cfg, x, *got[:4], got[4])
        torch.cuda.synchronize()
        assert got[4].cpu().view(torch.int32).item() == ref[4].cpu().view(torch.int32).item()
        for g, r in zip(got[:4], ref[:4]):
            if r is not None:
                assert torch.equal(g.cpu(), r.cpu())


def test_noalloc_empty_and_validation(fos):
    cfg = fos.make_config()
    t = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    fos.fos_quantize_noalloc(cfg, x, None, None, None, None, t)
    torch.cuda.synchronize()
    assert t.item() == 0.0
    L = fos.lib()
    fake = ctypes.c_void_p(t.data_ptr())
    assert L.fos_quantize_noalloc(ctypes.byref(cfg), fake, 16, 40, fake, fake, None, None, fake,
                                  None) == fos.FOS_E_SHAPE
    assert L.fos_quantize_noalloc(ctypes.byref(cfg), fake, 16, 32, None, fake, None, None, fake,
                                  None) == fos.FOS_E_NULL


def test_noalloc_on_a_side_stream(fos):
    """A call on another stream of the same GPU finds the same device's array."""
    cfg = fos.make_config(outputs=("row", "col"))
    x = W.random_bf16(256, 512, 40, "normal").to(DEV)
    ref = _outputs(256, 512, ("row", "col"))
    got = _outputs(256, 512, ("row", "col"))
    fos.fos_quantize(cfg, x, *ref[:4], ref[4])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        fos.fos_quantize_noalloc(cfg, x, *got[:4], got[4])
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert torch.equal(g.cpu(), r.cpu())
