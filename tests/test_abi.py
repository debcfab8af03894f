"""C ABI checks that need no GPU: the library loads, exports every entry point that
include/fos.h declares, and rejects bad arguments with the documented status before
any HIP call (the pointers passed here are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

from fp4_block_quantization_amd import fos

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "fos.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fos_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) >= 8
    out = subprocess.run(["nm", "-D", "--defined-only", fos.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fos_\w+)", out))
    for n in names:
        assert n in exported, n
        # the binding declares every signature (no implicit int conversions)
        assert getattr(fos.lib(), n).argtypes is not None, n


def test_ceiling_library_exports_and_validates():
    """libfos_ceiling.so (measured HBM ceilings for the benchmark) exports what
    include/fos_ceiling.h declares and rejects bad arguments before any launch."""
    text = open(os.path.join(ROOT, "include", "fos_ceiling.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(fos_[a-z_0-9]+)\s*\(", text)))
    path = os.path.join(os.path.dirname(fos.LIB_PATH), "libfos_ceiling.so")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (fos_\w+)", out))
    assert len(names) == 4 and set(names) <= exported
    L = ctypes.CDLL(path)
    L.fos_ceiling_granule.restype = ctypes.c_size_t
    g = L.fos_ceiling_granule()
    assert g == 8192
    P, SZ = ctypes.c_void_p, ctypes.c_size_t
    L.fos_ceiling_read.argtypes = [P, SZ, ctypes.c_uint32, P, P]
    L.fos_ceiling_copy.argtypes = [P, P, SZ, P]
    L.fos_ceiling_pattern.argtypes = [P, SZ, P, P, P]
    assert L.fos_ceiling_read(None, g, 0, FAKE, None) == 1
    assert L.fos_ceiling_read(FAKE, g + 16, 0, FAKE, None) == 2
    assert L.fos_ceiling_read(FAKE, 0, 0, FAKE, None) == 2
    assert L.fos_ceiling_copy(MIS, FAKE, g, None) == 3
    assert L.fos_ceiling_pattern(FAKE, g, ctypes.c_void_p(0x100004), FAKE, None) == 3
    assert L.fos_ceiling_pattern(FAKE, g, FAKE, None, None) == 1


# The calls the boundary must export: quantize, dequantize, the simulated quantized
# linear forward, the workspace query of quantize, and the status names.
BOUNDARY_CALLS = ("fos_quantize", "fos_dequantize", "fos_qlinear_fwd",
                  "fos_quantize_workspace_bytes", "fos_status_string")


def test_boundary_calls_exported_and_documented():
    names = declared_symbols()
    out = subprocess.run(["nm", "-D", "--defined-only", fos.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fos_\w+)", out))
    text = open(os.path.join(ROOT, "include", "fos.h")).read()
    for n in BOUNDARY_CALLS:
        assert n in names and n in exported, n
        # the comment right above the declaration cites a page section
        decl = re.search(r"/\*((?:(?!\*/).)*)\*/\s*(?:const char\*|size_t|fos_status)\s+" + n + r"\s*\(",
                         text, flags=re.S)
        assert decl is not None, n
        comment = re.sub(r"\s*\n\s*\*?\s*", " ", decl.group(1))    # one line of text
        if n != "fos_status_string":
            assert '"How FP4 works"' in comment or '"Four Over Six"' in comment, n
    assert fos.lib().fos_quantize_workspace_bytes() == fos.lib().fos_workspace_bytes()


def test_abi_version_and_strings():
    assert fos.ABI_VERSION == 2
    for s in range(7):
        assert fos.lib().fos_status_string(s).startswith(b"FOS_")
    assert fos.lib().fos_workspace_bytes() >= 8


FAKE = ctypes.c_void_p(0x100000)          # 16-byte aligned, never dereferenced
MIS = ctypes.c_void_p(0x100002)


def cfg(**kw):
    c = fos.make_config(**{k: v for k, v in kw.items() if k != "raw"})
    for k, v in kw.get("raw", {}).items():
        setattr(c, k, v)
    return c


def q(c, x=FAKE, rows=64, cols=64, rd=FAKE, rs=FAKE, cd=FAKE, cs=FAKE, t=FAKE, ws=FAKE, wsb=None):
    wsb = fos.lib().fos_workspace_bytes() if wsb is None else wsb
    return fos.lib().fos_quantize(ctypes.byref(c) if c is not None else None, x, rows, cols, rd, rs,
                                  cd, cs, t, ws, wsb, None)


@pytest.mark.parametrize("kw,args,want", [
    ({}, dict(cols=40), fos.FOS_E_SHAPE),
    ({}, dict(rows=-1), fos.FOS_E_SHAPE),
    (dict(outputs=("col",)), dict(rows=40), fos.FOS_E_SHAPE),
    (dict(block="2d"), dict(rows=24), fos.FOS_E_SHAPE),
    ({}, dict(x=None), fos.FOS_E_NULL),
    ({}, dict(x=MIS), fos.FOS_E_ALIGN),
    ({}, dict(rd=None), fos.FOS_E_NULL),
    ({}, dict(rd=ctypes.c_void_p(0x100004)), fos.FOS_E_ALIGN),
    (dict(outputs=("col",)), dict(cs=None), fos.FOS_E_NULL),
    ({}, dict(t=None), fos.FOS_E_NULL),
    ({}, dict(ws=None), fos.FOS_E_WORKSPACE),
    ({}, dict(wsb=4), fos.FOS_E_WORKSPACE),
    ({}, dict(ws=ctypes.c_void_p(0x100008)), fos.FOS_E_WORKSPACE),   # not 16-byte aligned
    (dict(raw={"rule": 7}), {}, fos.FOS_E_FLAGS),
    (dict(raw={"rounding": 3}), {}, fos.FOS_E_FLAGS),
    (dict(raw={"outputs": 0}), {}, fos.FOS_E_FLAGS),
    (dict(raw={"outputs": 4}), {}, fos.FOS_E_FLAGS),
    (dict(raw={"struct_size": 8}), {}, fos.FOS_E_FLAGS),
    (dict(block="2d", hadamard_seed=1), {}, fos.FOS_E_FLAGS),
    (dict(outputs=("row", "col"), hadamard_seed=1), {}, fos.FOS_E_FLAGS),
])
def test_quantize_validation(kw, args, want):
    assert q(cfg(**kw), **args) == want


def test_launch_grid_limit():
    """Shapes whose launch would exceed 2^32 - 1 work-items are rejected up front, with
    no kernel (not even the tensor-scale pass) launched."""
    L = fos.lib()
    f = FAKE
    # 2D tiles: (2^25 - 1) tile rows / 2 per workgroup -> 2^24 workgroups of 256
    assert q(cfg(block="2d"), rows=(1 << 29) - 16, cols=16) == fos.FOS_E_SHAPE
    # row-wise, one 16-value block per lane: 2^26 x 1040 -> 4,362,076,160 blocks in
    # 17,039,360 workgroups of 256 (more than (2^32 - 1) / 256)
    assert q(cfg(), rows=1 << 26, cols=1040) == fos.FOS_E_SHAPE
    # column-wise 128 x 64 tiles of a [2^31 - 16, 16] tensor -> 2^24 workgroups
    assert q(cfg(outputs=("col",)), rows=(1 << 31) - 16, cols=16) == fos.FOS_E_SHAPE
    t = ctypes.byref(cfg(outputs=("col",)))
    assert L.fos_quantize_scaled(t, f, (1 << 31) - 16, 16, f, f, f, f, f, None) == fos.FOS_E_SHAPE
    # a 2^20 x 2^20 output in 256 x 256 tiles -> 2^24 workgroups
    assert L.fos_qlinear_fwd(f, f, f, f, f, f, 1 << 20, 1 << 20, 64, f, None) == fos.FOS_E_SHAPE
    assert L.fos_mx_qlinear_fwd(f, f, f, f, 1 << 20, 1 << 20, 256, f, None) == fos.FOS_E_SHAPE
    # MXFP4 quantize: 512 blocks of 32 per workgroup
    assert L.fos_mx_quantize(f, 1 << 20, (1 << 18) + 32, f, f, None) == fos.FOS_E_SHAPE


def test_quantize_null_config():
    assert q(None) == fos.FOS_E_NULL


def test_dequantize_validation():
    L = fos.lib()
    assert L.fos_dequantize(FAKE, FAKE, FAKE, 4, 40, 0, FAKE, None) == fos.FOS_E_SHAPE
    assert L.fos_dequantize(FAKE, FAKE, FAKE, 4, 32, 5, FAKE, None) == fos.FOS_E_FLAGS
    assert L.fos_dequantize(None, FAKE, FAKE, 4, 32, 0, FAKE, None) == fos.FOS_E_NULL
    assert L.fos_dequantize(FAKE, FAKE, FAKE, 4, 32, 0, MIS, None) == fos.FOS_E_ALIGN
    assert L.fos_dequantize(None, None, None, 0, 32, 0, None, None) == fos.FOS_OK   # empty


def test_dequantize_hadamard_validation():
    L = fos.lib()
    f = FAKE
    assert L.fos_dequantize_hadamard(f, f, f, 4, 40, 1, 0, f, None) == fos.FOS_E_SHAPE
    assert L.fos_dequantize_hadamard(f, f, f, 4, 32, 1, 7, f, None) == fos.FOS_E_FLAGS
    assert L.fos_dequantize_hadamard(None, f, f, 4, 32, 1, 0, f, None) == fos.FOS_E_NULL
    assert L.fos_dequantize_hadamard(f, f, f, 4, 32, 1, 0, MIS, None) == fos.FOS_E_ALIGN
    assert L.fos_dequantize_hadamard(None, None, None, 0, 32, 1, 0, None, None) == fos.FOS_OK


def test_mx_validation():
    L = fos.lib()
    f = FAKE
    assert L.fos_mx_quantize(f, 4, 48, f, f, None) == fos.FOS_E_SHAPE          # cols % 32
    assert L.fos_mx_quantize(None, 4, 64, f, f, None) == fos.FOS_E_NULL
    assert L.fos_mx_quantize(MIS, 4, 64, f, f, None) == fos.FOS_E_ALIGN
    assert L.fos_mx_quantize(f, 4, 64, ctypes.c_void_p(0x100008), f, None) == fos.FOS_E_ALIGN
    assert L.fos_mx_quantize(None, 0, 64, None, None, None) == fos.FOS_OK
    assert L.fos_mx_dequantize(f, f, 4, 48, 0, f, None) == fos.FOS_E_SHAPE
    assert L.fos_mx_dequantize(f, f, 4, 64, 9, f, None) == fos.FOS_E_FLAGS
    assert L.fos_mx_dequantize(f, f, 4, 64, 0, MIS, None) == fos.FOS_E_ALIGN
    assert L.fos_mx_qlinear_fwd(f, f, f, f, 256, 256, 128, f, None) == fos.FOS_E_SHAPE   # K % 256
    assert L.fos_mx_qlinear_fwd(f, f, f, f, 0, 256, 256, f, None) == fos.FOS_E_SHAPE
    assert L.fos_mx_qlinear_fwd(None, f, f, f, 256, 256, 256, f, None) == fos.FOS_E_NULL
    assert L.fos_mx_qlinear_fwd(MIS, f, f, f, 256, 256, 256, f, None) == fos.FOS_E_ALIGN


def test_qlinear_validation():
    L = fos.lib()
    f = FAKE
    assert L.fos_qlinear_fwd(f, f, f, f, f, f, 256, 256, 100, f, None) == fos.FOS_E_SHAPE
    assert L.fos_qlinear_fwd(f, f, f, f, f, f, 0, 256, 256, f, None) == fos.FOS_E_SHAPE
    assert L.fos_qlinear_fwd(f, f, f, f, f, f, 256, 256, 32, f, None) == fos.FOS_E_SHAPE
    assert L.fos_qlinear_fwd(None, f, f, f, f, f, 256, 256, 256, f, None) == fos.FOS_E_NULL
    assert L.fos_qlinear_fwd(MIS, f, f, f, f, f, 256, 256, 256, f, None) == fos.FOS_E_ALIGN
    # a packed operand must fit one buffer resource (< 4 GiB)
    assert L.fos_qlinear_fwd(f, f, f, f, f, f, 1 << 20, 256, 1 << 13, f, None) == fos.FOS_E_SHAPE


def test_selftest_validation():
    L = fos.lib()
    assert L.fos_selftest_e4m3(None, None) == fos.FOS_E_NULL
    assert L.fos_selftest_e4m3(ctypes.c_void_p(0x100004), None) == fos.FOS_E_ALIGN
    assert L.fos_selftest_e2m1(None, None) == fos.FOS_E_NULL
    assert L.fos_selftest_e2m1(ctypes.c_void_p(0x100004), None) == fos.FOS_E_ALIGN
    assert L.fos_selftest_e2m1_sr(None, None) == fos.FOS_E_NULL
    assert L.fos_selftest_e2m1_sr(ctypes.c_void_p(0x100004), None) == fos.FOS_E_ALIGN
    assert L.fos_selftest_e2m1_sr_full(None, None) == fos.FOS_E_NULL
    assert L.fos_selftest_e2m1_sr_full(ctypes.c_void_p(0x100004), None) == fos.FOS_E_ALIGN


def test_qlinear_act_validation():
    """fos_qlinear_fwd_act checks the quantize options, the activation, the workspace
    and the GEMM operands before any launch."""
    L = fos.lib()
    f, z = FAKE, None
    M, N, K = 256, 256, 256
    need = L.fos_qlinear_act_workspace_bytes(M, K)
    assert need == M * K // 2 + M * K // 16 + L.fos_workspace_bytes()
    assert L.fos_qlinear_act_workspace_bytes(-1, 64) == 0
    big = ctypes.c_void_p(0x1000000)                        # 256-byte aligned

    def call(c=None, x=f, t=f, given=0, wd=f, wsc=f, wt=f, m=M, n=N, k=K, y=f, ws=big, wsb=need):
        c = cfg() if c is None else c
        return L.fos_qlinear_fwd_act(ctypes.byref(c), x, t, given, wd, wsc, wt, m, n, k, y, ws, wsb,
                                     None)
    assert call(c=cfg(outputs=("col",))) == fos.FOS_E_FLAGS
    assert call(c=cfg(outputs=("row", "col"))) == fos.FOS_E_FLAGS
    assert call(k=100) == fos.FOS_E_SHAPE                   # K % 16
    assert call(k=80) == fos.FOS_E_SHAPE                    # K % 64 (GEMM)
    assert call(m=0) == fos.FOS_E_SHAPE
    assert call(c=cfg(block="2d"), m=24) == fos.FOS_E_SHAPE
    assert call(x=z) == fos.FOS_E_NULL
    assert call(x=MIS) == fos.FOS_E_ALIGN
    assert call(t=z) == fos.FOS_E_NULL
    assert call(ws=z) == fos.FOS_E_WORKSPACE
    assert call(ws=ctypes.c_void_p(0x1000010)) == fos.FOS_E_WORKSPACE   # 16- but not 256-aligned
    assert call(wsb=need - 1) == fos.FOS_E_WORKSPACE
    assert call(wd=z) == fos.FOS_E_NULL
    assert call(y=z) == fos.FOS_E_NULL
    assert call(wd=MIS) == fos.FOS_E_ALIGN


def test_qlinear_bwd_validation():
    """All arguments are checked before either product launches; a skipped product's
    operands may be NULL."""
    L = fos.lib()
    f, z = FAKE, None
    ok3, no3 = [f, f, f], [z, z, z]
    # nothing requested
    assert L.fos_qlinear_bwd(*ok3, *ok3, *ok3, *ok3, 256, 256, 256, z, z, z) == fos.FOS_E_NULL
    # dX's inner dimension is N, dW's is M
    assert L.fos_qlinear_bwd(*ok3, *ok3, *ok3, *ok3, 256, 100, 256, f, z, z) == fos.FOS_E_SHAPE
    assert L.fos_qlinear_bwd(*ok3, *ok3, *ok3, *ok3, 100, 256, 256, z, f, z) == fos.FOS_E_SHAPE
    # a bad dW request fails validation even though dX alone would be fine
    assert L.fos_qlinear_bwd(*ok3, *ok3, *ok3, *ok3, 100, 256, 256, f, f, z) == fos.FOS_E_SHAPE
    # operands of the product that is computed must be present
    assert L.fos_qlinear_bwd(*ok3, *no3, *no3, *no3, 256, 256, 256, f, z, z) == fos.FOS_E_NULL
    assert L.fos_qlinear_bwd(*no3, *ok3, *no3, *no3, 256, 256, 256, z, f, z) == fos.FOS_E_NULL
    assert L.fos_qlinear_bwd(*ok3, *ok3, *ok3, MIS, f, f, 256, 256, 256, f, f, z) == fos.FOS_E_ALIGN


def test_tensor_scale_validation():
    L = fos.lib()
    c = cfg()
    assert L.fos_tensor_scale(ctypes.byref(c), FAKE, 16, 24, FAKE, FAKE, 1 << 14, None) == fos.FOS_E_SHAPE
    assert L.fos_tensor_scale(ctypes.byref(c), FAKE, 16, 32, None, FAKE, 4096, None) == fos.FOS_E_NULL
    assert L.fos_tensor_scale(ctypes.byref(c), FAKE, 16, 32, FAKE, FAKE, 8, None) == fos.FOS_E_WORKSPACE
    c2 = cfg(outputs=("col",), hadamard_seed=3)
    assert L.fos_tensor_scale(ctypes.byref(c2), FAKE, 24, 32, FAKE, FAKE, 1 << 14, None) == fos.FOS_E_SHAPE


def test_binding_rejects_host_records():
    """A record on the host would hand host addresses to the GPU: the binding refuses."""
    import torch
    q = fos.NVFP4Tensor(torch.zeros(4, 16, dtype=torch.uint8), torch.zeros(4, 2, dtype=torch.uint8),
                        torch.zeros(1))
    with pytest.raises(ValueError):
        fos.qlinear_fwd(q, q)
    with pytest.raises(ValueError):
        fos.dequantize(q)
    m = fos.MXFP4Tensor(torch.zeros(4, 16, dtype=torch.uint8), torch.zeros(4, 1, dtype=torch.uint8))
    with pytest.raises(ValueError):
        fos.mx_qlinear_fwd(m, m)
