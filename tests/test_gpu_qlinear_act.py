"""GPU parity of the quantized linear forward from a bf16 activation
(fos_qlinear_fwd_act): X is quantized inside the call, then multiplied with a weight
record.  The record the call leaves in its workspace must be bit-exact with the
oracle's quantization of X, and Y within 1e-3 normwise (plus the element-wise fp32
accumulation bound) of the fp64 reference built from the oracle's records of X and W.
Both inputs are seeded workloads; W's record is the oracle's, uploaded."""
import numpy as np
import pytest
import torch

from fp4_block_quantization_amd import workloads as W
from oracle import formats as F
from oracle import nvfp4 as N
from oracle.qlinear import qlinear_ref64
from test_gpu_parity import _qlinear_check, _sample_rows, assert_same_bytes, bits_of, to_gpu_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def fos():
    from fp4_block_quantization_amd import fos as mod
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return mod


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _weight_record(fos, wb, cfg):
    ow = N.quantize(wb, cfg)
    t = torch.tensor([ow["t"]], dtype=torch.float32, device=DEV)
    return ow, fos.NVFP4Tensor(_dev(ow["row_data"]), _dev(ow["row_scales"]), t)


def _kwargs(cfg):
    return dict(rule=cfg.rule, rounding=cfg.rounding, block=cfg.block,
                hadamard_seed=cfg.hadamard_seed if cfg.hadamard else None,
                sr_seed=cfg.sr_seed if cfg.rounding in ("sr", "sr_full") else None)


ACT_CFGS = {
    "4/6": N.Config(),
    "6": N.Config(rule="6"),
    "sr": N.Config(rounding="sr", sr_seed=4321),
    "sr_full": N.Config(rounding="sr_full", sr_seed=4323),
    "2d": N.Config(block="2d"),
    "rht": N.Config(hadamard=True, hadamard_seed=29),
}


@pytest.mark.parametrize("cfg_name", list(ACT_CFGS))
@pytest.mark.parametrize("m,n,k", [(256, 256, 64), (208, 520, 320), (1, 16, 64), (512, 768, 1024),
                                   (96, 136, 2048)])
def test_qlinear_act_matches_oracle(fos, cfg_name, m, n, k):
    cfg = ACT_CFGS[cfg_name]
    if cfg.block == "2d" and m % 16:
        pytest.skip("2D blocks need M % 16 == 0")
    xb = bits_of(W.random_bf16(m, k, 7 * m + k, "student_t", scale=0.5))
    wb = bits_of(W.random_bf16(n, k, 5 * n + k, "normal", scale=0.02))
    # the weight carries the same transform as X (it cancels in the product); 1D, RNE
    wcfg = N.Config(hadamard=cfg.hadamard, hadamard_seed=cfg.hadamard_seed)
    ow, wq = _weight_record(fos, wb, wcfg)
    y, xr = fos.qlinear_fwd_act(to_gpu_bf16(xb), wq, return_record=True, **_kwargs(cfg))
    torch.cuda.synchronize()
    ox = N.quantize(xb, cfg)
    assert np.float32(xr.tensor_scale.cpu()[0]).view(np.uint32) == np.float32(ox["t"]).view(np.uint32)
    assert_same_bytes(xr.data.cpu().numpy(), ox["row_data"], "x record data")
    assert_same_bytes(xr.scales.cpu().numpy(), ox["row_scales"], "x record scales")
    _qlinear_check(bits_of(y.cpu()), ox["row_data"], ox["row_scales"], ox["t"], ow["row_data"],
                   ow["row_scales"], ow["t"])


def test_qlinear_act_with_given_scale(fos):
    """A tensor scale supplied by the caller (here twice the tensor's own, as a delayed
    scale from an earlier, larger activation would be) is used as given and not
    overwritten; X is read once."""
    m, n, k = 320, 264, 768
    xb = bits_of(W.random_bf16(m, k, 91, "student_t", scale=0.5))
    wb = bits_of(W.random_bf16(n, k, 93, "normal", scale=0.02))
    ow, wq = _weight_record(fos, wb, N.Config())
    _, t_own = N.prepare(xb, N.Config())
    t_given = np.float32(2 * t_own)
    tg = torch.tensor([t_given], dtype=torch.float32, device=DEV)
    y, xr = fos.qlinear_fwd_act(to_gpu_bf16(xb), wq, x_tensor_scale=tg, return_record=True)
    torch.cuda.synchronize()
    assert np.float32(tg.cpu()[0]) == t_given
    ox = N.quantize(xb, N.Config(), t=t_given)
    assert_same_bytes(xr.data.cpu().numpy(), ox["row_data"], "x record data")
    assert_same_bytes(xr.scales.cpu().numpy(), ox["row_scales"], "x record scales")
    _qlinear_check(bits_of(y.cpu()), ox["row_data"], ox["row_scales"], t_given, ow["row_data"],
                   ow["row_scales"], ow["t"])


def test_qlinear_act_equals_quantize_then_qlinear(fos):
    """One call gives the bytes of fos_quantize followed by fos_qlinear_fwd."""
    m, n, k = 512, 384, 1280
    x = W.random_bf16(m, k, 101, "student_t").to(DEV)
    w = W.random_bf16(n, k, 103, "normal", scale=0.02).to(DEV)
    wq = fos.quantize(w)
    y1 = fos.qlinear_fwd_act(x, wq)
    y2 = fos.qlinear_fwd(fos.quantize(x), wq)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_qlinear_act_full_size_c5_sampled(fos):
    """The c5 layer (X 8192x4096 Student-t, W 12288x4096) from bf16 X: sampled rows of
    X's record bit-exact, sampled outputs within tolerance."""
    xb, wb = bits_of(W.make("c5_x")), bits_of(W.make("c5_w"))
    cfg = N.Config()
    _, tx = N.prepare(xb, cfg)
    _, tw = N.prepare(wb, cfg)
    wq = fos.quantize(to_gpu_bf16(wb))
    y, xr = fos.qlinear_fwd_act(to_gpu_bf16(xb), wq, return_record=True)
    torch.cuda.synchronize()
    assert np.float32(xr.tensor_scale.cpu()[0]).view(np.uint32) == np.float32(tx).view(np.uint32)
    rows = _sample_rows(xb.shape[0], 48, 11)
    cols = _sample_rows(wb.shape[0], 48, 12)
    ox = N.quantize_rows_sampled(xb, cfg, tx, rows)
    ow = N.quantize_rows_sampled(wb, cfg, tw, cols)
    assert_same_bytes(xr.data.cpu().numpy()[rows], ox["row_data"], "x record data")
    assert_same_bytes(xr.scales.cpu().numpy()[rows], ox["row_scales"], "x record scales")
    _qlinear_check(bits_of(y.cpu())[np.ix_(rows, cols)], ox["row_data"], ox["row_scales"], tx,
                   ow["row_data"], ow["row_scales"], tw)


def test_scale_pass_overlapped_with_the_previous_layer(fos):
    """Inference pipelining of the activation's tensor scale: while the previous layer's
    GEMM runs on the main stream, fos_tensor_scale(X) runs on a second stream; after an
    event wait the main stream runs fos_qlinear_fwd_act with the scale given, so X is
    read once.  The overlapped run must give X's record bit-exact with the oracle, Y
    within tolerance, and the previous layer's output unchanged."""
    m, n, k = 2048, 3072, 4096
    xb = bits_of(W.random_bf16(m, k, 111, "student_t", scale=0.5))
    pb = bits_of(W.random_bf16(m, k, 113, "student_t"))             # previous layer's input
    wb = bits_of(W.random_bf16(n, k, 115, "normal", scale=0.02))
    ow, wq = _weight_record(fos, wb, N.Config())
    pq = fos.quantize(to_gpu_bf16(pb))
    x = to_gpu_bf16(xb)
    y_prev_alone = fos.qlinear_fwd(pq, wq)
    torch.cuda.synchronize()

    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    t_x = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    side.wait_stream(main)                  # x, t_x and the records are ready
    y_prev = torch.empty_like(y_prev_alone)
    fos.qlinear_fwd(pq, wq, out=y_prev)                      # previous layer, main stream
    with torch.cuda.stream(side):
        fos.tensor_scale(x, out=t_x)                         # X's scale pass, side stream
        done = torch.cuda.Event()
        done.record(side)
    main.wait_event(done)
    y, xr = fos.qlinear_fwd_act(x, wq, x_tensor_scale=t_x, return_record=True)
    torch.cuda.synchronize()

    assert torch.equal(y_prev, y_prev_alone)
    ox = N.quantize(xb, N.Config())
    assert np.float32(t_x.cpu()[0]).view(np.uint32) == np.float32(ox["t"]).view(np.uint32)
    assert_same_bytes(xr.data.cpu().numpy(), ox["row_data"], "x record data")
    assert_same_bytes(xr.scales.cpu().numpy(), ox["row_scales"], "x record scales")
    rows = _sample_rows(m, 48, 13)
    cols = _sample_rows(n, 48, 14)
    sub = lambda o, r: {"row_data": o["row_data"][r], "row_scales": o["row_scales"][r]}
    sx, sw = sub(ox, rows), sub(ow, cols)
    _qlinear_check(bits_of(y.cpu())[np.ix_(rows, cols)], sx["row_data"], sx["row_scales"], ox["t"],
                   sw["row_data"], sw["row_scales"], ow["t"])
