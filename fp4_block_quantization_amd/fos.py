"""Thin ctypes binding of libfos.so (the C ABI declared in include/fos.h).

Argument marshalling only: every step of quantize / dequantize / qlinear runs in the
library's HIP kernels.  PyTorch provides device memory and the current HIP stream.
There is no fallback: if libfos.so is missing or fails to load, importing this
module raises.

Low-level functions carry the C names (fos_quantize, fos_dequantize, ...) and take
device tensors; ``quantize`` / ``dequantize`` / ``qlinear_fwd`` allocate the outputs.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple, Union

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfos.so")

FOS_OK, FOS_E_NULL, FOS_E_SHAPE, FOS_E_ALIGN, FOS_E_FLAGS, FOS_E_WORKSPACE, FOS_E_HIP = range(7)
FOS_RULE_4OVER6, FOS_RULE_6ONLY = 0, 1
FOS_ROUND_RNE, FOS_ROUND_STOCHASTIC, FOS_ROUND_STOCHASTIC_FULL = 0, 1, 2
FOS_BLOCK_1D, FOS_BLOCK_2D = 0, 1
FOS_OUT_ROWWISE, FOS_OUT_COLWISE = 1, 2
FOS_OUT_F32, FOS_OUT_BF16 = 0, 1


class FosError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_lib.fos_status_string(status).decode()} (status {status})")


class FosQuantConfig(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("rule", ctypes.c_uint32),
                ("rounding", ctypes.c_uint32), ("block", ctypes.c_uint32),
                ("outputs", ctypes.c_uint32), ("hadamard", ctypes.c_uint32),
                ("hadamard_seed", ctypes.c_uint64), ("sr_seed", ctypes.c_uint64)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m fp4_block_quantization_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    cfgp = ctypes.POINTER(FosQuantConfig)
    sigs = {
        "fos_abi_version": ([], ctypes.c_int),
        "fos_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "fos_quantize_workspace_bytes": ([], SZ),
        "fos_workspace_bytes": ([], SZ),
        "fos_tensor_scale": ([cfgp, P, I64, I64, P, P, SZ, P], ctypes.c_int),
        "fos_quantize_scaled": ([cfgp, P, I64, I64, P, P, P, P, P, P], ctypes.c_int),
        "fos_quantize": ([cfgp, P, I64, I64, P, P, P, P, P, P, SZ, P], ctypes.c_int),
        "fos_quantize_noalloc": ([cfgp, P, I64, I64, P, P, P, P, P, P], ctypes.c_int),
        "fos_selftest_e4m3": ([P, P], ctypes.c_int),
        "fos_selftest_e2m1": ([P, P], ctypes.c_int),
        "fos_selftest_e2m1_sr": ([P, P], ctypes.c_int),
        "fos_selftest_e2m1_sr_full": ([P, P], ctypes.c_int),
        "fos_dequantize": ([P, P, P, I64, I64, ctypes.c_int, P, P], ctypes.c_int),
        "fos_dequantize_hadamard": ([P, P, P, I64, I64, ctypes.c_uint64, ctypes.c_int, P, P],
                                    ctypes.c_int),
        "fos_qlinear_fwd": ([P, P, P, P, P, P, I64, I64, I64, P, P], ctypes.c_int),
        "fos_qlinear_bwd": ([P] * 12 + [I64, I64, I64, P, P, P], ctypes.c_int),
        "fos_qlinear_act_workspace_bytes": ([I64, I64], SZ),
        "fos_qlinear_fwd_act": ([cfgp, P, P, ctypes.c_int, P, P, P, I64, I64, I64, P, P, SZ, P],
                                ctypes.c_int),
        "fos_mx_quantize": ([P, I64, I64, P, P, P], ctypes.c_int),
        "fos_mx_dequantize": ([P, P, I64, I64, ctypes.c_int, P, P], ctypes.c_int),
        "fos_mx_qlinear_fwd": ([P, P, P, P, I64, I64, I64, P, P], ctypes.c_int),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()
ABI_VERSION = _lib.fos_abi_version()


def lib() -> ctypes.CDLL:
    return _lib


# ---------------------------------------------------------------- marshalling helpers

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(status: int, what: str):
    if status != FOS_OK:
        raise FosError(status, what)


def make_config(rule: str = "4/6", rounding: str = "rne", block: str = "1d",
                outputs: Sequence[str] = ("row",), hadamard_seed: Optional[int] = None,
                sr_seed: Optional[int] = None) -> FosQuantConfig:
    rules = {"4/6": FOS_RULE_4OVER6, "6": FOS_RULE_6ONLY}
    roundings = {"rne": FOS_ROUND_RNE, "sr": FOS_ROUND_STOCHASTIC,
                 "sr_full": FOS_ROUND_STOCHASTIC_FULL}
    blocks = {"1d": FOS_BLOCK_1D, "2d": FOS_BLOCK_2D}
    out = 0
    for o in outputs:
        out |= {"row": FOS_OUT_ROWWISE, "col": FOS_OUT_COLWISE}[o]
    if rounding in ("sr", "sr_full") and sr_seed is None:
        raise ValueError("stochastic rounding needs sr_seed")
    return FosQuantConfig(ctypes.sizeof(FosQuantConfig), rules[rule], roundings[rounding],
                          blocks[block], out, 0 if hadamard_seed is None else 1,
                          0 if hadamard_seed is None else int(hadamard_seed) & (2 ** 64 - 1),
                          0 if sr_seed is None else int(sr_seed) & (2 ** 64 - 1))


_workspaces = {}


def workspace(device: torch.device) -> torch.Tensor:
    """Scratch workspace for the current stream of ``device`` (one per stream, so
    that calls on different streams never share one; its contents are scratch)."""
    device = torch.device(device)
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None:
        ws = torch.zeros(int(_lib.fos_quantize_workspace_bytes()), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


# ---------------------------------------------------------------- C-named wrappers

def fos_tensor_scale(cfg: FosQuantConfig, x: torch.Tensor, tensor_scale: torch.Tensor,
                     ws: Optional[torch.Tensor] = None) -> None:
    ws = workspace(x.device) if ws is None else ws
    _check(_lib.fos_tensor_scale(ctypes.byref(cfg), _ptr(x), x.shape[0], x.shape[1],
                                 _ptr(tensor_scale), _ptr(ws), ws.numel(), _stream(x.device)),
           "fos_tensor_scale")


def fos_quantize_scaled(cfg: FosQuantConfig, x: torch.Tensor, tensor_scale: torch.Tensor,
                        row_data=None, row_scales=None, col_data=None, col_scales=None) -> None:
    _check(_lib.fos_quantize_scaled(ctypes.byref(cfg), _ptr(x), x.shape[0], x.shape[1],
                                    _ptr(tensor_scale), _ptr(row_data), _ptr(row_scales),
                                    _ptr(col_data), _ptr(col_scales), _stream(x.device)),
           "fos_quantize_scaled")


def fos_quantize(cfg: FosQuantConfig, x: torch.Tensor, row_data, row_scales, col_data,
                 col_scales, tensor_scale: torch.Tensor,
                 ws: Optional[torch.Tensor] = None) -> None:
    ws = workspace(x.device) if ws is None else ws
    _check(_lib.fos_quantize(ctypes.byref(cfg), _ptr(x), x.shape[0], x.shape[1],
                             _ptr(row_data), _ptr(row_scales), _ptr(col_data), _ptr(col_scales),
                             _ptr(tensor_scale), _ptr(ws), ws.numel(), _stream(x.device)),
           "fos_quantize")


def fos_quantize_noalloc(cfg: FosQuantConfig, x: torch.Tensor, row_data, row_scales, col_data,
                         col_scales, tensor_scale: torch.Tensor) -> None:
    """fos_quantize without a workspace: the library's own per-GPU scratch array holds
    the tensor-scale pass's partial maxima (calls on one GPU must not overlap)."""
    _check(_lib.fos_quantize_noalloc(ctypes.byref(cfg), _ptr(x), x.shape[0], x.shape[1],
                                     _ptr(row_data), _ptr(row_scales), _ptr(col_data),
                                     _ptr(col_scales), _ptr(tensor_scale), _stream(x.device)),
           "fos_quantize_noalloc")


def selftest_e4m3(device="cuda:0") -> int:
    """Number of fp32 values in [0, 448] whose hardware E4M3 conversion (used by the
    quantize kernels for the block scales) differs from the bit-level rule; 0 on a
    correct device."""
    n = torch.zeros(1, dtype=torch.int64, device=device)
    _check(_lib.fos_selftest_e4m3(_ptr(n), _stream(n.device)), "fos_selftest_e4m3")
    return int(n.item())


def selftest_e2m1(device="cuda:0") -> int:
    """Number of finite fp32 values whose hardware E2M1 conversion (used by the quantize
    kernels for the element codes) differs from the rounding rule; 0 on a correct
    device."""
    n = torch.zeros(1, dtype=torch.int64, device=device)
    _check(_lib.fos_selftest_e2m1(_ptr(n), _stream(n.device)), "fos_selftest_e2m1")
    return int(n.item())


def selftest_e2m1_sr(device="cuda:0") -> int:
    """Number of (finite fp32 value, draw byte, pair position) cases where the
    hardware stochastic rounding to E2M1, under the operands the quantize kernels
    build from their draws, differs from the draw rule; 0 on a correct device."""
    n = torch.zeros(1, dtype=torch.int64, device=device)
    _check(_lib.fos_selftest_e2m1_sr(_ptr(n), _stream(n.device)), "fos_selftest_e2m1_sr")
    return int(n.item())


def selftest_e2m1_sr_full(device="cuda:0") -> int:
    """Number of disagreements at the rounding boundary of the full-resolution
    stochastic rounding (every finite fp32 value, both pair positions); 0 on a
    correct device."""
    n = torch.zeros(1, dtype=torch.int64, device=device)
    _check(_lib.fos_selftest_e2m1_sr_full(_ptr(n), _stream(n.device)), "fos_selftest_e2m1_sr_full")
    return int(n.item())


def fos_dequantize(data: torch.Tensor, scales: torch.Tensor, tensor_scale: torch.Tensor,
                   rows: int, cols: int, out: torch.Tensor) -> None:
    dt = {torch.float32: FOS_OUT_F32, torch.bfloat16: FOS_OUT_BF16}[out.dtype]
    _check(_lib.fos_dequantize(_ptr(data), _ptr(scales), _ptr(tensor_scale), rows, cols, dt,
                               _ptr(out), _stream(out.device)), "fos_dequantize")


def fos_dequantize_hadamard(data: torch.Tensor, scales: torch.Tensor, tensor_scale: torch.Tensor,
                            rows: int, cols: int, hadamard_seed: int, out: torch.Tensor) -> None:
    dt = {torch.float32: FOS_OUT_F32, torch.bfloat16: FOS_OUT_BF16}[out.dtype]
    _check(_lib.fos_dequantize_hadamard(_ptr(data), _ptr(scales), _ptr(tensor_scale), rows, cols,
                                        hadamard_seed, dt, _ptr(out), _stream(out.device)),
           "fos_dequantize_hadamard")


def fos_qlinear_fwd(x_data, x_scales, x_t, w_data, w_scales, w_t, M: int, N: int, K: int,
                    y: torch.Tensor) -> None:
    _check(_lib.fos_qlinear_fwd(_ptr(x_data), _ptr(x_scales), _ptr(x_t), _ptr(w_data),
                                _ptr(w_scales), _ptr(w_t), M, N, K, _ptr(y), _stream(y.device)),
           "fos_qlinear_fwd")


def fos_qlinear_bwd(dy, dyt, xt, wt, M: int, N: int, K: int, dx: Optional[torch.Tensor],
                    dw: Optional[torch.Tensor]) -> None:
    """dy, dyt, xt, wt: (data, scales, tensor_scale) triples (a skipped product's
    operands may be None)."""
    def trip(r):
        return [_ptr(v) for v in r] if r is not None else [_ptr(None)] * 3
    dev = (dx if dx is not None else dw).device
    _check(_lib.fos_qlinear_bwd(*trip(dy), *trip(dyt), *trip(xt), *trip(wt), M, N, K, _ptr(dx),
                                _ptr(dw), _stream(dev)), "fos_qlinear_bwd")


def fos_qlinear_fwd_act(cfg: FosQuantConfig, x: torch.Tensor, x_t: torch.Tensor,
                        x_scale_given: bool, w_data, w_scales, w_t, N: int, y: torch.Tensor,
                        ws: torch.Tensor) -> None:
    M, K = x.shape
    _check(_lib.fos_qlinear_fwd_act(ctypes.byref(cfg), _ptr(x), _ptr(x_t), int(bool(x_scale_given)),
                                    _ptr(w_data), _ptr(w_scales), _ptr(w_t), M, N, K, _ptr(y),
                                    _ptr(ws), ws.numel(), _stream(x.device)),
           "fos_qlinear_fwd_act")


# ---------------------------------------------------------------- tensor-level API

@dataclass
class NVFP4Tensor:
    """One NVFP4 record: data [R, C/2] nibbles, scales [R, C/16] E4M3 bytes, and the
    per-tensor fp32 scale (device tensor of one element).  ``layout`` is "row" for
    the row-wise record of X and "col" for the record of X^T."""
    data: torch.Tensor
    scales: torch.Tensor
    tensor_scale: torch.Tensor
    layout: str = "row"
    block: str = "1d"
    hadamard_seed: Optional[int] = None

    @property
    def shape(self) -> Tuple[int, int]:
        return (self.data.shape[0], self.data.shape[1] * 2)


def _check_input(x: torch.Tensor):
    if x.dim() != 2 or x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D bfloat16 CUDA tensor")


def _check_record(q, *others):
    """A record's tensors must be contiguous CUDA tensors on one device (the library
    dereferences them on the GPU), with the shapes the layout implies."""
    dev = q.data.device
    tensors = [q.data, q.scales] + ([q.tensor_scale] if hasattr(q, "tensor_scale") else [])
    for o in others:
        tensors += [o.data, o.scales] + ([o.tensor_scale] if hasattr(o, "tensor_scale") else [])
    for t in tensors:
        if not t.is_cuda or t.device != dev or not t.is_contiguous():
            raise ValueError("record tensors must be contiguous CUDA tensors on one device")
    for r in (q,) + others:
        if r.data.dtype != torch.uint8 or r.scales.dtype != torch.uint8 or r.data.dim() != 2:
            raise ValueError("record data and scales must be 2-D uint8 tensors")
        block = 32 if not hasattr(r, "tensor_scale") else 16
        R, C = r.shape
        if tuple(r.scales.shape) != (R, C // block):
            raise ValueError(f"scales must be [{R}, {C // block}]")


def tensor_scale(x: torch.Tensor, hadamard_seed: Optional[int] = None,
                 outputs: Sequence[str] = ("row",), out: Optional[torch.Tensor] = None
                 ) -> torch.Tensor:
    """The per-tensor FP32 scale t of x (device fp32 [1]), on the current stream;
    ``out``: optional destination."""
    _check_input(x)
    cfg = make_config(outputs=outputs, hadamard_seed=hadamard_seed)
    t = out if out is not None else torch.empty(1, dtype=torch.float32, device=x.device)
    if t.dtype != torch.float32 or t.numel() != 1 or t.device != x.device:
        raise ValueError("out must be a one-element fp32 tensor on x's device")
    fos_tensor_scale(cfg, x, t)
    return t


def quantize(x: torch.Tensor, rule: str = "4/6", rounding: str = "rne", block: str = "1d",
             outputs: Sequence[str] = ("row",), hadamard_seed: Optional[int] = None,
             sr_seed: Optional[int] = None, tensor_scale: Optional[torch.Tensor] = None
             ) -> Union[NVFP4Tensor, Tuple[NVFP4Tensor, NVFP4Tensor]]:
    """4/6 NVFP4 quantization of a bf16 [R, C] tensor.  Returns the row-wise record,
    the column-wise record (quantization of X^T), or both as (row, col).  With
    ``tensor_scale`` given (device fp32 [1]) the amax pass is skipped."""
    _check_input(x)
    cfg = make_config(rule, rounding, block, outputs, hadamard_seed, sr_seed)
    R, C = x.shape
    dev = x.device
    u8 = dict(dtype=torch.uint8, device=dev)
    rd = rs = cd = cs = None
    if "row" in outputs:
        rd, rs = torch.empty(R, C // 2, **u8), torch.empty(R, C // 16, **u8)
    if "col" in outputs:
        cd, cs = torch.empty(C, R // 2, **u8), torch.empty(C, R // 16, **u8)
    if tensor_scale is None:
        t = torch.empty(1, dtype=torch.float32, device=dev)
        fos_quantize(cfg, x, rd, rs, cd, cs, t)
    else:
        t = tensor_scale
        fos_quantize_scaled(cfg, x, t, rd, rs, cd, cs)
    res = []
    if rd is not None:
        res.append(NVFP4Tensor(rd, rs, t, "row", block, hadamard_seed))
    if cd is not None:
        res.append(NVFP4Tensor(cd, cs, t, "col", block, hadamard_seed))
    return res[0] if len(res) == 1 else tuple(res)


def dequantize(q: NVFP4Tensor, dtype: torch.dtype = torch.float32,
               inverse_hadamard: bool = False) -> torch.Tensor:
    """Dequantize a record ([R, C] as stored).  With ``inverse_hadamard`` a record made
    with the random Hadamard transform is returned to the original basis."""
    _check_record(q)
    R, C = q.shape
    out = torch.empty(R, C, dtype=dtype, device=q.data.device)
    if inverse_hadamard:
        if q.hadamard_seed is None:
            raise ValueError("the record was not made with the Hadamard transform")
        fos_dequantize_hadamard(q.data, q.scales, q.tensor_scale, R, C, q.hadamard_seed, out)
    else:
        fos_dequantize(q.data, q.scales, q.tensor_scale, R, C, out)
    return out


def qlinear_fwd(xq: NVFP4Tensor, wq: NVFP4Tensor, out: Optional[torch.Tensor] = None
                ) -> torch.Tensor:
    """Y = deq(A) deq(B)^T in bf16 for two records blocked along their shared inner
    dimension: A [M, K], B [N, K] as stored (a column-wise record of W is the record
    of W^T; 2D records carry one scale per 16 values too).  ``out``: optional bf16
    [M, N] destination."""
    _check_record(xq, wq)
    M, K = xq.shape
    N, K2 = wq.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    y = out if out is not None else torch.empty(M, N, dtype=torch.bfloat16,
                                                device=xq.data.device)
    if y.shape != (M, N) or y.dtype != torch.bfloat16 or not y.is_contiguous():
        raise ValueError("out must be a contiguous bf16 [M, N] tensor")
    fos_qlinear_fwd(xq.data, xq.scales, xq.tensor_scale, wq.data, wq.scales, wq.tensor_scale,
                    M, N, K, y)
    return y


def qlinear_act_workspace(M: int, K: int, device) -> torch.Tensor:
    """A workspace for qlinear_fwd_act on X [M, K] (torch allocations are 256-byte
    aligned)."""
    n = int(_lib.fos_qlinear_act_workspace_bytes(M, K))
    if n == 0:
        raise ValueError("unsupported activation shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def act_record(ws: torch.Tensor, M: int, K: int, tensor_scale: torch.Tensor,
               block: str = "1d", hadamard_seed: Optional[int] = None) -> NVFP4Tensor:
    """Views of the record of X that qlinear_fwd_act leaves in its workspace."""
    up = lambda v: (v + 255) // 256 * 256
    nd, ns = M * K // 2, M * K // 16
    data = ws[:nd].view(M, K // 2)
    scales = ws[up(nd):up(nd) + ns].view(M, K // 16)
    return NVFP4Tensor(data, scales, tensor_scale, "row", block, hadamard_seed)


def qlinear_fwd_act(x: torch.Tensor, wq: NVFP4Tensor, rule: str = "4/6", rounding: str = "rne",
                    block: str = "1d", hadamard_seed: Optional[int] = None,
                    sr_seed: Optional[int] = None, x_tensor_scale: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, return_record: bool = False):
    """Y = deq(Q(X)) deq(Wq)^T in bf16 from a bf16 activation X [M, K] and a weight
    record Wq [N, K]: X is quantized with the given options inside the call.  With
    ``x_tensor_scale`` (device fp32 [1], e.g. a delayed scale) X is read once;
    otherwise its tensor scale is computed.  ``return_record`` also returns X's
    record (views of a fresh workspace)."""
    _check_input(x)
    _check_record(wq)
    M, K = x.shape
    N, K2 = wq.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    if wq.data.device != x.device:
        raise ValueError("x and the weight record are on different devices")
    cfg = make_config(rule, rounding, block, ("row",), hadamard_seed, sr_seed)
    y = out if out is not None else torch.empty(M, N, dtype=torch.bfloat16, device=x.device)
    if y.shape != (M, N) or y.dtype != torch.bfloat16 or not y.is_contiguous():
        raise ValueError("out must be a contiguous bf16 [M, N] tensor")
    given = x_tensor_scale is not None
    t = x_tensor_scale if given else torch.empty(1, dtype=torch.float32, device=x.device)
    ws = qlinear_act_workspace(M, K, x.device)
    fos_qlinear_fwd_act(cfg, x, t, given, wq.data, wq.scales, wq.tensor_scale, N, y, ws)
    if return_record:
        return y, act_record(ws, M, K, t, block, hadamard_seed)
    return y


def qlinear_bwd(dyq: Optional[NVFP4Tensor], dyq_t: Optional[NVFP4Tensor],
                xq_t: Optional[NVFP4Tensor], wq_t: Optional[NVFP4Tensor],
                need_dx: bool = True, need_dw: bool = True
                ) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
    """Backward of Y = X W^T from NVFP4 records: dX = deq(dY) deq(W^T)^T and
    dW = deq(dY^T) deq(X^T)^T (bf16).  dyq: row-wise record of dY [M, N]; dyq_t,
    xq_t, wq_t: column-wise records of dY, X and W (records of dY^T [N, M], X^T [K, M],
    W^T [K, N])."""
    if not (need_dx or need_dw):
        raise ValueError("nothing to compute")
    used = ([dyq, wq_t] if need_dx else []) + ([dyq_t, xq_t] if need_dw else [])
    _check_record(*used)
    if need_dx:
        M, N = dyq.shape
        K, N2 = wq_t.shape
        if N2 != N:
            raise ValueError("dY and W disagree on N")
    if need_dw:
        N3, M3 = dyq_t.shape
        K3, M4 = xq_t.shape
        if M3 != M4:
            raise ValueError("dY and X disagree on M")
        if need_dx and (N3 != N or M3 != M or K3 != K):
            raise ValueError("inconsistent shapes")
        M, N, K = M3, N3, K3
    ref = dyq if need_dx else dyq_t
    dev = ref.data.device
    dx = torch.empty(M, K, dtype=torch.bfloat16, device=dev) if need_dx else None
    dw = torch.empty(N, K, dtype=torch.bfloat16, device=dev) if need_dw else None
    trip = lambda q: (q.data, q.scales, q.tensor_scale) if q is not None else None
    fos_qlinear_bwd(trip(dyq) if need_dx else None, trip(dyq_t) if need_dw else None,
                    trip(xq_t) if need_dw else None, trip(wq_t) if need_dx else None,
                    M, N, K, dx, dw)
    return dx, dw


# ---------------------------------------------------------------- MXFP4

@dataclass
class MXFP4Tensor:
    """One MXFP4 record: data [R, C/2] nibbles and scales [R, C/32] E8M0 bytes."""
    data: torch.Tensor
    scales: torch.Tensor

    @property
    def shape(self) -> Tuple[int, int]:
        return (self.data.shape[0], self.data.shape[1] * 2)


def mx_quantize(x: torch.Tensor) -> MXFP4Tensor:
    """MXFP4 quantization of a bf16 [R, C] tensor (C % 32 == 0)."""
    _check_input(x)
    R, C = x.shape
    u8 = dict(dtype=torch.uint8, device=x.device)
    data, scales = torch.empty(R, C // 2, **u8), torch.empty(R, C // 32, **u8)
    _check(_lib.fos_mx_quantize(_ptr(x), R, C, _ptr(data), _ptr(scales), _stream(x.device)),
           "fos_mx_quantize")
    return MXFP4Tensor(data, scales)


def mx_dequantize(q: MXFP4Tensor, dtype: torch.dtype = torch.float32) -> torch.Tensor:
    _check_record(q)
    R, C = q.shape
    out = torch.empty(R, C, dtype=dtype, device=q.data.device)
    dt = {torch.float32: FOS_OUT_F32, torch.bfloat16: FOS_OUT_BF16}[dtype]
    _check(_lib.fos_mx_dequantize(_ptr(q.data), _ptr(q.scales), R, C, dt, _ptr(out),
                                  _stream(out.device)), "fos_mx_dequantize")
    return out


def mx_qlinear_fwd(aq: MXFP4Tensor, bq: MXFP4Tensor, out: Optional[torch.Tensor] = None
                   ) -> torch.Tensor:
    """Y = deq(A) deq(B)^T in bf16 on the FP4 matrix cores; A [M, K], B [N, K]."""
    _check_record(aq, bq)
    M, K = aq.shape
    N, K2 = bq.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    y = out if out is not None else torch.empty(M, N, dtype=torch.bfloat16, device=aq.data.device)
    if y.shape != (M, N) or y.dtype != torch.bfloat16 or not y.is_contiguous():
        raise ValueError("out must be a contiguous bf16 [M, N] tensor")
    _check(_lib.fos_mx_qlinear_fwd(_ptr(aq.data), _ptr(aq.scales), _ptr(bq.data), _ptr(bq.scales),
                                   M, N, K, _ptr(y), _stream(y.device)), "fos_mx_qlinear_fwd")
    return y

