"""Benchmark of the 4/6 NVFP4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME] [--no-cpu]

A step is one fos_quantize call (tensor-scale pass + fused 4/6 quantize kernel) on the
weight workload 4096x12288 bf16 (1D 16-value row blocks, 4/6, round-to-nearest-even),
the configuration the headline metric is quoted on.  Inputs are resident in HBM
before timing; three input/output sets (> 256 MB of inputs) rotate so that no call
finds its input in the 256 MB Infinity Cache.  Before the first timed loop the step
runs back to back for half a second (untimed) so that the GPU is at its steady
clock; then W warm-up steps and K timed steps.  Times come from HIP events on the
stream the kernels are launched on (torch's current stream).

Printed: ONE JSON line with the headline (quantize GB/s of algorithmic bytes), the
roofline of the dominant kernel (the quantize kernel timed alone, given the tensor
scale: K calls issued back to back from pre-marshalled C-ABI calls between two HIP
events, and the same K calls captured in a HIP graph and replayed; the smaller
per-call time of the two, both reported), the CPU oracle timed on a bounded sample,
and the other hot-path rows
(column-wise, Hadamard + stochastic rounding, 2D, dequantize, qlinear TFLOP/s from
quantized and from bf16 activations, backward, MXFP4).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense fp16/bf16 MFMA, published (2.5 PFLOP/s)
FP4_MFMA_PEAK_TFLOPS = 10066.3  # MI355X dense fp4 MFMA, published (10.1 PFLOP/s)
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "fp4_block_quantization_amd", "csrc", f)
                  for f in ("quantize.hip", "device_common.hpp")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()


def quant_bytes(rows, cols, n_out=1):
    n = rows * cols
    return 2 * n + n_out * (n // 2 + n // 16) + 4


def settle(fn, rotate, seconds):
    """Run fn(i) back to back for `seconds` of wall time, untimed.  An idle GPU starts
    at a low clock and takes tens of milliseconds of sustained work to reach its
    steady one; without this the first timed loop of a fresh process can read
    half the steady rate."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn(i % rotate)
            i += 1
        torch.cuda.synchronize()


def time_loop(fn, steps, warmup, rotate):
    """Average ms per call of fn(i) over `steps` calls after `warmup`, i rotating."""
    import torch
    for i in range(warmup):
        fn(i % rotate)
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(steps):
        fn(i % rotate)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def graph_loop(make_fn, steps, warmup, rotate):
    """Average ms per call of `steps` calls captured in one HIP graph (torch.cuda.CUDAGraph)
    and replayed, so that the GPU runs the kernels back to back without waiting for the
    host to launch each one.  make_fn(stream) returns fn(i) issuing call i on `stream`."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn = make_fn(side)
        for i in range(max(3, warmup)):
            fn(i % rotate)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn = make_fn(torch.cuda.current_stream())
        for i in range(steps):
            fn(i % rotate)
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    g.replay()
    e.record()
    torch.cuda.synchronize()
    del g
    return s.elapsed_time(e) / steps


def _vp(t):
    import ctypes
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


class QuantCase:
    """Rotating input/output sets for one quantize configuration.  The C ABI calls
    are pre-marshalled (pointers, sizes, stream) so that the Python side issues each
    call in about a microsecond and the GPU is never starved between launches."""

    def __init__(self, fos, x_cpu, cfg_kw, sets):
        import ctypes
        import torch
        self.fos = fos
        self.cfg = fos.make_config(**cfg_kw)
        self.outputs = cfg_kw.get("outputs", ("row",))
        R, C = x_cpu.shape
        self.R, self.C = R, C
        dev = "cuda:0"
        self.x = [x_cpu.to(dev) for _ in range(sets)]
        u8 = dict(dtype=torch.uint8, device=dev)
        self.out = []
        for _ in range(sets):
            rd = rs = cd = cs = None
            if "row" in self.outputs:
                rd, rs = torch.empty(R, C // 2, **u8), torch.empty(R, C // 16, **u8)
            if "col" in self.outputs:
                cd, cs = torch.empty(C, R // 2, **u8), torch.empty(C, R // 16, **u8)
            self.out.append((rd, rs, cd, cs))
        self.t = [torch.zeros(1, dtype=torch.float32, device=dev) for _ in range(sets)]
        self.ws = fos.workspace(dev)
        self.sets = sets
        lib = fos.lib()
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        cref = ctypes.byref(self.cfg)
        nws = self.ws.numel()
        self._q, self._qs, self._ts = lib.fos_quantize, lib.fos_quantize_scaled, lib.fos_tensor_scale
        self.args_q, self.args_qs, self.args_ts = [], [], []
        for i in range(sets):
            rd, rs, cd, cs = self.out[i]
            x, t = _vp(self.x[i]), _vp(self.t[i])
            self.args_q.append((cref, x, R, C, _vp(rd), _vp(rs), _vp(cd), _vp(cs), t,
                                _vp(self.ws), nws, stream))
            self.args_qs.append((cref, x, R, C, t, _vp(rd), _vp(rs), _vp(cd), _vp(cs), stream))
            self.args_ts.append((cref, x, R, C, t, _vp(self.ws), nws, stream))
        self.bad = 0

    def on_stream(self, stream, scaled=True):
        """fn(i) issuing call i (fos_quantize_scaled, or fos_quantize) on `stream`."""
        import ctypes
        h = ctypes.c_void_p(stream.cuda_stream)
        args = [a[:-1] + (h,) for a in (self.args_qs if scaled else self.args_q)]
        f = self._qs if scaled else self._q

        def fn(i):
            self.bad |= f(*args[i])
        return fn

    def step(self, i):
        self.bad |= self._q(*self.args_q[i])

    def scaled(self, i):
        self.bad |= self._qs(*self.args_qs[i])

    def scale_only(self, i):
        self.bad |= self._ts(*self.args_ts[i])


def bench_quant(fos, name, x_cpu, cfg_kw, steps, warmup, n_out=1, settle_s=0.2):
    R, C = x_cpu.shape
    sets = min(8, max(3, -(-300 * 2 ** 20 // (2 * R * C))))   # > 256 MB of inputs rotate
    case = QuantCase(fos, x_cpu, cfg_kw, sets)
    if settle_s > 0:
        settle(case.step, sets, settle_s)
    ms = time_loop(case.step, steps, warmup, sets)
    # the same steps replayed from a HIP graph: a check that the eager step is not bound
    # by the host's launches (reported beside it, not used for the headline)
    try:
        ms_step_graph = graph_loop(lambda st: case.on_stream(st, scaled=False), steps, warmup, sets)
    except RuntimeError as exc:
        log(f"{name}: step graph capture failed ({exc})")
        ms_step_graph = None
    ms_k_b2b = time_loop(case.scaled, steps, warmup, sets)
    try:
        ms_k_graph = graph_loop(case.on_stream, steps, warmup, sets)
    except RuntimeError as exc:    # capture unavailable: back-to-back calls only
        log(f"{name}: graph capture failed ({exc})")
        ms_k_graph = None
    # Both are the per-call time of the same K calls; each has its own overhead (host
    # jitter between eager launches, per-node work in the graph), so the kernel's time
    # is the smaller of the two.
    ms_k = ms_k_b2b if ms_k_graph is None else min(ms_k_b2b, ms_k_graph)
    ms_a = time_loop(case.scale_only, steps, warmup, sets)
    if case.bad:
        raise RuntimeError(f"{name}: a fos call returned an error status")
    b = quant_bytes(R, C, n_out)
    row = {"workload": name, "shape": [R, C], "options": {k: (list(v) if isinstance(v, tuple) else v)
                                                          for k, v in cfg_kw.items()},
           "bytes": b, "ms_step": ms, "GBps_step": b / ms / 1e6, "ms_step_graph_replay": ms_step_graph,
           "frac_step": b / ms / 1e6 / HBM_PEAK_GBS,
           "ms_quant_kernel": ms_k, "GBps_quant_kernel": b / ms_k / 1e6,
           "frac_quant_kernel": b / ms_k / 1e6 / HBM_PEAK_GBS,
           "quant_kernel_timing": "min(back_to_back_calls, hip_graph_replay)",
           "ms_quant_kernel_back_to_back_calls": ms_k_b2b,
           "ms_quant_kernel_graph_replay": ms_k_graph,
           "ms_scale_kernel": ms_a, "GBps_scale_kernel": 2 * R * C / ms_a / 1e6}
    del case
    return row


def bench_dequant(fos, x_cpu, steps, warmup):
    import ctypes
    import torch
    R, C = x_cpu.shape
    dev = "cuda:0"
    q = fos.quantize(x_cpu.to(dev))
    lib = fos.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    rows = {}
    for dt, name, ob, code in ((torch.bfloat16, "bf16", 2, fos.FOS_OUT_BF16),
                               (torch.float32, "f32", 4, fos.FOS_OUT_F32)):
        sets = 3
        outs = [torch.empty(R, C, dtype=dt, device=dev) for _ in range(sets)]
        datas = [q.data.clone() for _ in range(sets)]
        scs = [q.scales.clone() for _ in range(sets)]
        args = [(_vp(datas[i]), _vp(scs[i]), _vp(q.tensor_scale), R, C, code, _vp(outs[i]), stream)
                for i in range(sets)]
        f = lib.fos_dequantize
        bad = [0]

        def fn(i):
            bad[0] |= f(*args[i])
        ms = time_loop(fn, steps, warmup, sets)
        if bad[0]:
            raise RuntimeError("fos_dequantize returned an error status")
        b = R * C // 2 + R * C // 16 + 4 + ob * R * C
        rows[name] = {"bytes": b, "ms": ms, "GBps": b / ms / 1e6, "frac": b / ms / 1e6 / HBM_PEAK_GBS}
        del outs
    return rows


def bench_dequant_hadamard(fos, x_cpu, steps, warmup):
    """Dequantize + inverse Hadamard transform of the c4a record (bf16 out)."""
    import ctypes
    import torch
    R, C = x_cpu.shape
    dev = "cuda:0"
    q = fos.quantize(x_cpu.to(dev), hadamard_seed=0, rounding="sr", sr_seed=1234)
    lib = fos.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    sets = 3
    outs = [torch.empty(R, C, dtype=torch.bfloat16, device=dev) for _ in range(sets)]
    datas = [q.data.clone() for _ in range(sets)]
    scs = [q.scales.clone() for _ in range(sets)]
    args = [(_vp(datas[i]), _vp(scs[i]), _vp(q.tensor_scale), R, C, 0, fos.FOS_OUT_BF16,
             _vp(outs[i]), stream) for i in range(sets)]
    f = lib.fos_dequantize_hadamard
    bad = [0]

    def fn(i):
        bad[0] |= f(*args[i])
    ms = time_loop(fn, steps, warmup, sets)
    if bad[0]:
        raise RuntimeError("fos_dequantize_hadamard returned an error status")
    b = R * C // 2 + R * C // 16 + 4 + 2 * R * C
    return {"bytes": b, "ms": ms, "GBps": b / ms / 1e6, "frac": b / ms / 1e6 / HBM_PEAK_GBS}


def bench_qlinear(fos, x_cpu, w_cpu, steps, warmup):
    import torch
    dev = "cuda:0"
    xq = fos.quantize(x_cpu.to(dev))
    wq = fos.quantize(w_cpu.to(dev))
    M, K = xq.shape
    N = wq.shape[0]
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)

    def fn(i):
        fos.fos_qlinear_fwd(xq.data, xq.scales, xq.tensor_scale, wq.data, wq.scales,
                            wq.tensor_scale, M, N, K, y)
    # the GPU's clocks settle over the first tens of milliseconds of sustained MFMA
    # work, so the untimed warm-up is about 20 ms of GEMMs
    ms = time_loop(fn, max(10, steps // 2), max(30, warmup), 1)
    flops = 2 * M * N * K
    row = {"shape": [M, N, K], "flop": flops, "ms": ms, "TFLOPs": flops / ms / 1e9,
           "frac": flops / ms / 1e9 / FP16_MFMA_PEAK_TFLOPS}
    # reference point, not part of the path: torch's dense bf16 matmul of the unquantized
    # operands at the same shape (the vendor GEMM, no dequantization), same timing loop
    xb = x_cpu.to(dev)
    wt = w_cpu.to(dev).t().contiguous()
    yb = torch.empty(M, N, dtype=torch.bfloat16, device=dev)

    def fb(i):
        torch.matmul(xb, wt, out=yb)
    ms_b = time_loop(fb, max(10, steps // 2), max(30, warmup), 1)
    row["torch_bf16_matmul_reference"] = {"ms": ms_b, "TFLOPs": flops / ms_b / 1e9,
                                          "frac": flops / ms_b / 1e9 / FP16_MFMA_PEAK_TFLOPS}
    return row


def bench_qlinear_act(fos, x_cpu, w_cpu, steps, warmup):
    """The c5 layer from a bf16 activation (fos_qlinear_fwd_act): X's quantization and
    the GEMM in one call, with X's tensor scale computed in the call (two passes over
    X) or given (one pass)."""
    import ctypes
    import torch
    dev = "cuda:0"
    lib = fos.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    x = x_cpu.to(dev)
    wq = fos.quantize(w_cpu.to(dev))
    M, K = x.shape
    N = wq.shape[0]
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    ws = fos.qlinear_act_workspace(M, K, dev)
    t = torch.zeros(1, dtype=torch.float32, device=dev)
    cfg = fos.make_config()
    f = lib.fos_qlinear_fwd_act
    flops = 2 * M * N * K
    out = {"shape": [M, N, K], "flop": flops}
    for name, given in (("scale_computed", 0), ("scale_given", 1)):
        args = (ctypes.byref(cfg), _vp(x), _vp(t), given, _vp(wq.data), _vp(wq.scales),
                _vp(wq.tensor_scale), M, N, K, _vp(y), _vp(ws), ws.numel(), stream)
        bad = [0]

        def fn(i):
            bad[0] |= f(*args)
        ms = time_loop(fn, max(10, steps // 2), max(15, warmup), 1)
        if bad[0]:
            raise RuntimeError("fos_qlinear_fwd_act returned an error status")
        out[name] = {"ms": ms, "TFLOPs": flops / ms / 1e9,
                     "frac": flops / ms / 1e9 / FP16_MFMA_PEAK_TFLOPS}
    return out


def bench_qlinear_overlap(fos, x_cpu, w_cpu, steps, warmup):
    """The inference pipelining of the activation's tensor scale, on the c5 shapes: a
    previous layer's GEMM (fos_qlinear_fwd on quantized input) followed by this layer
    from bf16 X (fos_qlinear_fwd_act with X's scale given, so X is read once).
    sequential: X's scale pass, the previous GEMM and this layer on one stream.
    overlapped: the scale pass on a second stream beside the previous GEMM; this layer
    waits for it on an event.  per_layer = overlapped - the previous GEMM alone."""
    import torch
    dev = "cuda:0"
    x = x_cpu.to(dev)
    wq = fos.quantize(w_cpu.to(dev))
    pq = fos.quantize(x)                          # the previous layer's quantized input
    M, K = x.shape
    N = wq.shape[0]
    y_prev = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    t = torch.zeros(1, dtype=torch.float32, device=dev)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        fos.tensor_scale(x, out=t)               # the side stream's workspace, made once
    torch.cuda.synchronize()

    def prev_gemm(i):
        fos.qlinear_fwd(pq, wq, out=y_prev)

    def sequential(i):
        fos.tensor_scale(x, out=t)
        fos.qlinear_fwd(pq, wq, out=y_prev)
        fos.qlinear_fwd_act(x, wq, x_tensor_scale=t, out=y)

    def overlapped(i):
        side.wait_stream(main)                   # t is free once the last layer read it
        with torch.cuda.stream(side):
            fos.tensor_scale(x, out=t)
            ev = torch.cuda.Event()
            ev.record(side)
        fos.qlinear_fwd(pq, wq, out=y_prev)
        main.wait_event(ev)
        fos.qlinear_fwd_act(x, wq, x_tensor_scale=t, out=y)

    n = max(6, steps // 4)
    ms_prev = time_loop(prev_gemm, n, max(10, warmup), 1)
    ms_seq = time_loop(sequential, n, max(5, warmup), 1)
    ms_ovl = time_loop(overlapped, n, max(5, warmup), 1)
    flops = 2 * M * N * K
    return {"shape": [M, N, K], "ms_previous_gemm": ms_prev, "ms_two_layers_sequential": ms_seq,
            "ms_two_layers_overlapped": ms_ovl, "ms_layer_overlapped": ms_ovl - ms_prev,
            "TFLOPs_layer_overlapped": flops / (ms_ovl - ms_prev) / 1e9,
            "ms_scale_pass_hidden": ms_seq - ms_ovl}


def bench_qlinear_bwd(fos, x_cpu, w_cpu, dy_cpu, steps, warmup):
    """Backward products of the c5 layer: dX = deq(dY) deq(W^T)^T (inner 12288) and
    dW = deq(dY^T) deq(X^T)^T (inner 8192), from training-style records: dY row and
    column-wise with stochastic rounding, X column-wise, W column-wise in 2D blocks."""
    import torch
    dev = "cuda:0"
    gq, gqt = fos.quantize(dy_cpu.to(dev), outputs=("row", "col"), rounding="sr", sr_seed=1234)
    xqt = fos.quantize(x_cpu.to(dev), outputs=("col",))
    wqt = fos.quantize(w_cpu.to(dev), outputs=("col",), block="2d")
    M, N = gq.shape
    K = xqt.shape[0]
    dx = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    dw = torch.empty(N, K, dtype=torch.bfloat16, device=dev)
    trip = lambda q: (q.data, q.scales, q.tensor_scale)

    def fn(i):
        fos.fos_qlinear_bwd(trip(gq), trip(gqt), trip(xqt), trip(wqt), M, N, K, dx, dw)
    ms = time_loop(fn, max(10, steps // 2), max(15, warmup), 1)
    flops = 2 * (2 * M * N * K)
    return {"shapes": {"dX": [M, K, N], "dW": [N, K, M]}, "flop": flops, "ms": ms,
            "TFLOPs": flops / ms / 1e9, "frac": flops / ms / 1e9 / FP16_MFMA_PEAK_TFLOPS}


def bench_mx(fos, x_cpu, w_cpu, x2_cpu, steps, warmup):
    """MXFP4: quantize the c2 weight (GB/s) and the c5 layer on the FP4 matrix cores."""
    import ctypes
    import torch
    dev = "cuda:0"
    lib = fos.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    R, C = x2_cpu.shape
    sets = 3
    xs = [x2_cpu.to(dev) for _ in range(sets)]
    u8 = dict(dtype=torch.uint8, device=dev)
    outs = [(torch.empty(R, C // 2, **u8), torch.empty(R, C // 32, **u8)) for _ in range(sets)]
    args = [(_vp(xs[i]), R, C, _vp(outs[i][0]), _vp(outs[i][1]), stream) for i in range(sets)]
    f = lib.fos_mx_quantize
    bad = [0]

    def fq(i):
        bad[0] |= f(*args[i])
    ms_q = time_loop(fq, steps, warmup, sets)
    qb = 2 * R * C + R * C // 2 + R * C // 32
    outs16 = [torch.empty(R, C, dtype=torch.bfloat16, device=dev) for _ in range(sets)]
    dargs = [(_vp(outs[i][0]), _vp(outs[i][1]), R, C, fos.FOS_OUT_BF16, _vp(outs16[i]), stream)
             for i in range(sets)]
    fd_ = lib.fos_mx_dequantize

    def fd(i):
        bad[0] |= fd_(*dargs[i])
    ms_d = time_loop(fd, steps, warmup, sets)
    db = R * C // 2 + R * C // 32 + 2 * R * C
    del outs16
    aq = fos.mx_quantize(x_cpu.to(dev))
    bq = fos.mx_quantize(w_cpu.to(dev))
    M, K = aq.shape
    N = bq.shape[0]
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    g = lib.fos_mx_qlinear_fwd
    gargs = (_vp(aq.data), _vp(aq.scales), _vp(bq.data), _vp(bq.scales), M, N, K, _vp(y), stream)

    def fg(i):
        bad[0] |= g(*gargs)
    ms_g = time_loop(fg, max(10, steps // 2), max(30, warmup), 1)
    if bad[0]:
        raise RuntimeError("an MXFP4 call returned an error status")
    flops = 2 * M * N * K
    gemm = {"shape": [M, N, K], "flop": flops, "ms": ms_g, "TFLOPs": flops / ms_g / 1e9,
            "frac_fp4_peak": flops / ms_g / 1e9 / FP4_MFMA_PEAK_TFLOPS}
    # reference point, not part of the path: torch's scaled matmul (the vendor MXFP4 GEMM)
    # on the same two records, same timing loop; null where this torch cannot run it
    try:
        a4, b4 = aq.data.view(torch.float4_e2m1fn_x2), bq.data.view(torch.float4_e2m1fn_x2)
        sa, sb = aq.scales.view(torch.float8_e8m0fnu), bq.scales.view(torch.float8_e8m0fnu)
        yt = torch._scaled_mm(a4, b4.t(), sa.flatten(), sb.flatten(), out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        rel = ((yt.float() - y.float()).norm() / y.float().norm()).item()

        def ft(i):
            torch._scaled_mm(a4, b4.t(), sa.flatten(), sb.flatten(), out_dtype=torch.bfloat16)
        ms_t = time_loop(ft, max(10, steps // 2), max(30, warmup), 1)
        gemm["torch_scaled_mm_reference"] = {"ms": ms_t, "TFLOPs": flops / ms_t / 1e9,
                                             "frac_fp4_peak": flops / ms_t / 1e9 / FP4_MFMA_PEAK_TFLOPS,
                                             "rel_diff_vs_ours": rel}
    except (RuntimeError, AttributeError, TypeError) as exc:
        log(f"torch scaled matmul reference unavailable: {exc}")
        gemm["torch_scaled_mm_reference"] = None
    return {"quantize_c2": {"bytes": qb, "ms": ms_q, "GBps": qb / ms_q / 1e6,
                            "frac": qb / ms_q / 1e6 / HBM_PEAK_GBS},
            "dequantize_c2_bf16": {"bytes": db, "ms": ms_d, "GBps": db / ms_d / 1e6,
                                   "frac": db / ms_d / 1e6 / HBM_PEAK_GBS},
            "gemm_c5": gemm}


CEILING_LIB = os.path.join(ROOT, "fp4_block_quantization_amd", "libfos_ceiling.so")


def _ceiling_lib():
    import ctypes
    lib = ctypes.CDLL(CEILING_LIB)
    P, SZ = ctypes.c_void_p, ctypes.c_size_t
    lib.fos_ceiling_read.argtypes = [P, SZ, ctypes.c_uint32, P, P]
    lib.fos_ceiling_copy.argtypes = [P, P, SZ, P]
    lib.fos_ceiling_pattern.argtypes = [P, SZ, P, P, P]
    return lib


class Ceilings:
    """Hand-written kernels (libfos_ceiling.so) that move the c2 quantize kernel's
    bytes without computing: a streaming read of the 100.7 MB input, a copy of it
    (read + write), and the row-wise quantize kernel's exact traffic (read 32 bytes,
    write 8 + 1 per 16 values).  Three input sets (> 256 MB) rotate."""

    def __init__(self, nbytes, sets=3):
        import ctypes
        import torch
        self.lib = _ceiling_lib()
        dev = "cuda:0"
        self.n = nbytes
        u8 = dict(dtype=torch.uint8, device=dev)
        self.x = [torch.randint(0, 255, (nbytes,), **u8) for _ in range(sets)]
        self.y = [torch.empty(nbytes, **u8) for _ in range(sets)]
        self.y8 = [torch.empty(nbytes // 4, **u8) for _ in range(sets)]
        self.y1 = [torch.empty(nbytes // 32, **u8) for _ in range(sets)]
        self.sink = torch.zeros(1, dtype=torch.int32, device=dev)
        self.stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        self.sets = sets
        self.bad = 0

    def read(self, i):
        self.bad |= self.lib.fos_ceiling_read(_vp(self.x[i]), self.n, 0x9E3779B9, _vp(self.sink),
                                              self.stream)

    def copy(self, i):
        self.bad |= self.lib.fos_ceiling_copy(_vp(self.x[i]), _vp(self.y[i]), self.n, self.stream)

    def pattern(self, i):
        self.bad |= self.lib.fos_ceiling_pattern(_vp(self.x[i]), self.n, _vp(self.y8[i]),
                                                 _vp(self.y1[i]), self.stream)


def bench_ceilings(nbytes, steps, warmup):
    c = Ceilings(nbytes)
    rows = {}
    for name, fn, moved in (("read", c.read, nbytes), ("copy", c.copy, 2 * nbytes),
                            ("c2_quantize_pattern", c.pattern, nbytes + nbytes // 4 + nbytes // 32)):
        settle(fn, c.sets, 0.1)
        ms = time_loop(fn, steps, warmup, c.sets)
        rows[name] = {"bytes": moved, "ms": ms, "GBps": moved / ms / 1e6,
                      "frac": moved / ms / 1e6 / HBM_PEAK_GBS}
    if c.bad:
        raise RuntimeError("a ceiling kernel returned an error status")
    del c
    return rows


def bench_step_ceiling(fos, x_cpu, steps, warmup):
    """The two-pass step against its own ceiling: the scale pass (fos_tensor_scale) followed
    by the pattern kernel (the quantize kernel's exact traffic, no arithmetic), and followed
    by the quantize kernel (fos_quantize_scaled), on the same rotating inputs.  The second
    pass of each sees its input partly in the memory-side cache, as inside the step."""
    import ctypes
    import torch
    dev = "cuda:0"
    R, C = x_cpu.shape
    case = QuantCase(fos, x_cpu, {}, 3)
    cl = _ceiling_lib()
    nb = 2 * R * C
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    bad = [0]

    def pattern(i):
        rd, rs = case.out[i][0], case.out[i][1]
        bad[0] |= cl.fos_ceiling_pattern(_vp(case.x[i]), nb, _vp(rd), _vp(rs), stream)

    def scale_then_pattern(i):
        case.scale_only(i)
        pattern(i)

    def scale_then_quantize(i):
        case.scale_only(i)
        case.scaled(i)
    out = {}
    for name, fn in (("scale_pass", case.scale_only), ("scale_pass_then_pattern", scale_then_pattern),
                     ("scale_pass_then_quantize", scale_then_quantize)):
        settle(fn, case.sets, 0.1)
        out["ms_" + name] = time_loop(fn, steps, warmup, case.sets)
    if bad[0] or case.bad:
        raise RuntimeError("a step-ceiling call returned an error status")
    out["ms_pattern_in_step"] = out["ms_scale_pass_then_pattern"] - out["ms_scale_pass"]
    out["ms_quantize_in_step"] = out["ms_scale_pass_then_quantize"] - out["ms_scale_pass"]
    out["quantize_over_pattern_in_step"] = out["ms_quantize_in_step"] / out["ms_pattern_in_step"]
    del case
    return out


def cpu_baseline(x_cpu, rows_sample):
    """The oracle, as it stands, on a slice of the weight workload (its own amax)."""
    import numpy as np
    import torch
    from oracle import nvfp4 as N
    bits = x_cpu[:rows_sample].contiguous().view(torch.int16).numpy().view(np.uint16)
    t0 = time.perf_counter()
    N.quantize(bits, N.Config())
    dt = time.perf_counter() - t0
    b = quant_bytes(rows_sample, x_cpu.shape[1])
    return {"value": b / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle quantize of {rows_sample} rows of the 4096x12288 weight "
                      f"({rows_sample * x_cpu.shape[1]} values, tensor scale included), "
                      f"{dt:.1f} s of single-threaded NumPy"}


_MC_BITS = None


def _mc_quantize(args):
    import numpy as np
    from oracle import nvfp4 as N
    lo, hi, t = args
    N.quantize(_MC_BITS[lo:hi], N.Config(), t=np.float32(t))
    return hi - lo


def cpu_baselines_extra(x_cpu, x5_cpu, w5_cpu, workers):
    """Reported CPU baselines beside the single-core one: the oracle row-chunked over
    `workers` processes (tensor scale in the parent), and the pages' own fallback for
    the quantized linear, an fp32 matmul over dequantized operands on the CPU."""
    import multiprocessing as mp
    import numpy as np
    import torch
    from oracle import nvfp4 as N
    global _MC_BITS
    bits = x_cpu.contiguous().view(torch.int16).numpy().view(np.uint16)
    t0 = time.perf_counter()
    _, t = N.prepare(bits, N.Config())
    _MC_BITS = bits
    R = bits.shape[0]
    edges = np.linspace(0, R, 4 * workers + 1).astype(int)
    with mp.get_context("fork").Pool(workers) as pool:
        done = sum(pool.map(_mc_quantize, [(int(a), int(b), float(t)) for a, b in zip(edges[:-1], edges[1:])]))
    dt = time.perf_counter() - t0
    assert done == R
    b = quant_bytes(R, bits.shape[1])
    mc = {"value": b / dt / 1e9, "unit": "GB/s", "cores": workers, "kind": "oracle",
          "sample": f"oracle quantize of the whole 4096x12288 weight, row chunks over {workers} "
                    f"processes, {dt:.1f} s"}
    # fp32 matmul fallback on a 1024-row slice of X against all of W (c5 shapes; the
    # operand values do not change the time of a dense fp32 matmul)
    xs = x5_cpu[:1024].float().contiguous()
    ws = w5_cpu.float().contiguous()
    torch.matmul(xs[:64], ws.T)
    t0 = time.perf_counter()
    reps = 3
    for _ in range(reps):
        torch.matmul(xs, ws.T)
    dt = (time.perf_counter() - t0) / reps
    flops = 2 * xs.shape[0] * ws.shape[0] * xs.shape[1]
    mm = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": torch.get_num_threads(),
          "kind": "fp32 matmul (the pages' CPU fallback)",
          "sample": f"torch.matmul fp32 [1024, 4096] x [4096, 12288] on the CPU, {dt * 1e3:.0f} ms"}
    return mc, mm


def traffic_for(kernel: str):
    try:
        rec = json.load(open(PMC_FILE))[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != source_hash():
        return None
    return rec.get("hbm_bytes_per_dispatch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default=None,
                    help="profiling aid: run one piece (c2_kernel, c3_kernel, c4a_kernel, c4a_full_kernel, c4b_kernel; "
                         "the same with _step for the whole step; "
                         "c2_dequant_bf16, c2_dequant_f32, c2_mx_dequant_bf16, "
                         "c4a_dequant_hadamard_bf16, c5_qlinear, c5_qlinear_act, "
                         "c5_qlinear_act_given, c5_mx_gemm, copy, ceiling_read, ceiling_copy, "
                         "ceiling_pattern) and exit")
    ap.add_argument("--settle", type=float, default=0.0,
                    help="with --only <config>_kernel or _step: run it back to back for this many "
                         "seconds first, so that the clock has settled (adds dispatches to a trace)")
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the multi-GPU "
              "path (per-shard tensor scale, one 4-byte max all-reduce) is not built.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from fp4_block_quantization_amd import workloads as W

    x2 = W.make("c2")
    # CPU baselines first, before anything touches the GPU: the multi-process one forks
    # workers, which must not inherit an initialised GPU runtime.
    cpu = None
    cpu_rows = {}
    if not args.no_cpu and args.only is None:
        log("CPU oracle baseline ...")
        cpu = cpu_baseline(x2, x2.shape[0])
        workers = max(1, min(16, os.cpu_count() or 1))   # one GPU's share of the host cores
        log(f"CPU oracle on {workers} processes, CPU fp32 matmul ...")
        mc, mm = cpu_baselines_extra(x2, W.make("c5_x"), W.make("c5_w"), workers)
        cpu_rows = {"cpu_oracle_multicore": mc, "cpu_fp32_matmul_c5_slice": mm}

    from fp4_block_quantization_amd import fos
    log(f"device: {torch.cuda.get_device_name(0)}")

    if args.only is not None:
        if args.only == "c5_qlinear":
            xq = fos.quantize(W.make("c5_x").to("cuda:0"))
            wq = fos.quantize(W.make("c5_w").to("cuda:0"))
            y = fos.qlinear_fwd(xq, wq)
            for _ in range(args.steps):
                fos.qlinear_fwd(xq, wq, out=y)
            torch.cuda.synchronize()
            log(f"ran c5_qlinear x{args.steps}")
            return
        if args.only == "c5_mx_gemm":
            aq = fos.mx_quantize(W.make("c5_x").to("cuda:0"))
            bq = fos.mx_quantize(W.make("c5_w").to("cuda:0"))
            y = fos.mx_qlinear_fwd(aq, bq)
            for _ in range(args.steps):
                fos.mx_qlinear_fwd(aq, bq, out=y)
            torch.cuda.synchronize()
            log(f"ran c5_mx_gemm x{args.steps}")
            return
        if args.only in ("c5_qlinear_act", "c5_qlinear_act_given"):
            wq = fos.quantize(W.make("c5_w").to("cuda:0"))
            x = W.make("c5_x").to("cuda:0")
            t = fos.tensor_scale(x) if args.only.endswith("given") else None
            y = fos.qlinear_fwd_act(x, wq, x_tensor_scale=t)
            for _ in range(args.steps):
                fos.qlinear_fwd_act(x, wq, x_tensor_scale=t, out=y)
            torch.cuda.synchronize()
            log(f"ran {args.only} x{args.steps}")
            return
        if args.only in ("c2_dequant_bf16", "c2_dequant_f32", "c2_mx_dequant_bf16",
                         "c4a_dequant_hadamard_bf16"):
            dt = torch.float32 if args.only == "c2_dequant_f32" else torch.bfloat16
            if args.only == "c2_mx_dequant_bf16":
                q = fos.mx_quantize(x2.to("cuda:0"))
                run = lambda: fos.mx_dequantize(q, dt)
            elif args.only == "c4a_dequant_hadamard_bf16":
                q = fos.quantize(W.make("c4a").to("cuda:0"), hadamard_seed=0, rounding="sr",
                                 sr_seed=1234)
                run = lambda: fos.dequantize(q, dt, inverse_hadamard=True)
            else:
                q = fos.quantize(x2.to("cuda:0"))
                run = lambda: fos.dequantize(q, dt)
            for _ in range(args.steps):
                run()
            torch.cuda.synchronize()
            log(f"ran {args.only} x{args.steps}")
            return
        if args.only == "copy":
            a = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device="cuda:0")
            b = torch.empty_like(a)
            for _ in range(args.steps):
                b.copy_(a)
            torch.cuda.synchronize()
            log("copy: 268435456 bytes per dispatch")
            return
        if args.only in ("ceiling_read", "ceiling_copy", "ceiling_pattern"):
            c = Ceilings(2 * x2.numel())
            fn = getattr(c, args.only.split("_", 1)[1])
            for i in range(args.steps):
                fn(i % c.sets)
            torch.cuda.synchronize()
            if c.bad:
                raise RuntimeError("a ceiling kernel returned an error status")
            log(f"ran {args.only} x{args.steps} on {c.n} input bytes")
            return
        kernels = {"c2_kernel": ("c2", {}), "c2_step": ("c2", {}),
                   "c3_kernel": ("c3", {"outputs": ("row", "col")}),
                   "c4a_kernel": ("c4a", {"hadamard_seed": 0, "rounding": "sr", "sr_seed": 1234}),
                   "c4a_full_kernel": ("c4a", {"hadamard_seed": 0, "rounding": "sr_full",
                                               "sr_seed": 1234}),
                   "c4b_kernel": ("c4b", {"block": "2d"})}
        # <config>_step: the whole step (scale pass + quantize) of that configuration
        kernels.update({k.replace("_kernel", "_step"): v for k, v in kernels.items()
                        if k.endswith("_kernel")})
        if args.only not in kernels:
            raise SystemExit(f"unknown --only {args.only}")
        name, kw = kernels[args.only]
        case = QuantCase(fos, x2 if name == "c2" else W.make(name), kw, 3)
        fn = case.step if args.only.endswith("_step") else case.scaled
        case.step(0); case.step(1); case.step(2)
        if args.settle > 0:
            settle(fn, 3, args.settle)
        for i in range(args.steps):
            fn(i % 3)
        torch.cuda.synchronize()
        log(f"ran {args.only} x{args.steps}")
        return

    log("C2 weight quantize ...")
    head = bench_quant(fos, "c2 weight 4096x12288, 1D rows, 4/6, RNE", x2, {}, args.steps, args.warmup,
                       settle_s=0.5)
    rows = {"c2_quantize": head}
    log(json.dumps(head))
    log("C2 dequantize ...")
    rows["c2_dequantize"] = bench_dequant(fos, x2, args.steps, args.warmup)
    log("C1 ...")
    rows["c1_quantize"] = bench_quant(fos, "c1 256x256, 1D rows, 4/6, RNE", W.make("c1"), {},
                                      args.steps, args.warmup)
    log("C3 ...")
    rows["c3_row_col"] = bench_quant(fos, "c3 activation 8192x4096, row + column outputs",
                                     W.make("c3"), {"outputs": ("row", "col")}, args.steps,
                                     args.warmup, n_out=2)
    log("C4a ...")
    rows["c4a_rht_sr"] = bench_quant(fos, "c4a gradient 8192x4096, Hadamard + stochastic rounding",
                                     W.make("c4a"), {"hadamard_seed": 0, "rounding": "sr",
                                                     "sr_seed": 1234}, args.steps, args.warmup)
    log("C4a with full-resolution stochastic rounding ...")
    rows["c4a_rht_sr_full"] = bench_quant(fos, "c4a gradient 8192x4096, Hadamard + full-resolution "
                                          "stochastic rounding", W.make("c4a"),
                                          {"hadamard_seed": 0, "rounding": "sr_full",
                                           "sr_seed": 1234}, args.steps, args.warmup)
    log("C4a inverse-Hadamard dequantize ...")
    rows["c4a_dequantize_hadamard_bf16"] = bench_dequant_hadamard(fos, W.make("c4a"), args.steps,
                                                                  args.warmup)
    log("C4b ...")
    rows["c4b_2d"] = bench_quant(fos, "c4b weight 12288x4096, 2D 16x16", W.make("c4b"),
                                 {"block": "2d"}, args.steps, args.warmup)
    log("HBM ceilings ...")
    rows["hbm_ceilings_c2_bytes"] = bench_ceilings(2 * x2.numel(), args.steps, args.warmup)
    log(json.dumps(rows["hbm_ceilings_c2_bytes"]))
    log("C2 two-pass step against its ceiling ...")
    rows["c2_step_ceiling"] = bench_step_ceiling(fos, x2, args.steps, args.warmup)
    log(json.dumps(rows["c2_step_ceiling"]))
    log("C5 qlinear ...")
    rows["c5_qlinear"] = bench_qlinear(fos, W.make("c5_x"), W.make("c5_w"), args.steps, args.warmup)
    log(json.dumps(rows["c5_qlinear"]))
    log("C5 qlinear from bf16 X ...")
    rows["c5_qlinear_act"] = bench_qlinear_act(fos, W.make("c5_x"), W.make("c5_w"), args.steps,
                                               args.warmup)
    log(json.dumps(rows["c5_qlinear_act"]))
    log("C5 layer with the scale pass overlapped ...")
    rows["c5_qlinear_act_overlap"] = bench_qlinear_overlap(fos, W.make("c5_x"), W.make("c5_w"),
                                                           args.steps, args.warmup)
    log(json.dumps(rows["c5_qlinear_act_overlap"]))
    log("C5 qlinear backward ...")
    rows["c5_qlinear_bwd"] = bench_qlinear_bwd(fos, W.make("c5_x"), W.make("c5_w"),
                                               W.make("c5_dy"), args.steps, args.warmup)
    log(json.dumps(rows["c5_qlinear_bwd"]))

    log("MXFP4 ...")
    rows["mxfp4"] = bench_mx(fos, W.make("c5_x"), W.make("c5_w"), x2, args.steps, args.warmup)
    log(json.dumps(rows["mxfp4"]))

    rows.update(cpu_rows)

    kernel_gbps = head["GBps_quant_kernel"]
    out = {
        "metric": "4/6 NVFP4 quantize GB/s (bf16 in) & % HBM peak; qlinear fwd TFLOP/s",
        "value": round(head["GBps_step"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "4/6 NVFP4 quantize of a 4096x12288 bf16 weight "
                               "(N(0,0.02), 0.1% x50 outliers), 1D 16-value row blocks, RNE",
                   "rows": 4096, "cols": 12288, "algorithmic_bytes_per_step": head["bytes"],
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "quant_rows_kernel (fos_quantize_scaled)",
                     "achieved": round(kernel_gbps, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kernel_gbps / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for("quant_rows_kernel")},
        "cpu_baseline": cpu,
        "qlinear_TFLOPs": round(rows["c5_qlinear"]["TFLOPs"], 1),
        "qlinear_frac_fp16_mfma_peak": round(rows["c5_qlinear"]["frac"], 4),
        "rows": rows,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
