"""Four Over Six (4/6) NVFP4 block quantization for AMD MI355X (gfx950).

The compute path is libfos.so (hand-written HIP kernels behind the C ABI of
include/fos.h); ``fp4_block_quantization_amd.fos`` is its ctypes binding and raises
on import if the library is missing.  ``workloads`` holds the seeded synthetic
inputs.  Tensor-level entry points (quantize, dequantize, qlinear_fwd, ...) are
re-exported lazily from ``fos``.
"""
_EXPORTS = ("quantize", "dequantize", "qlinear_fwd", "tensor_scale", "NVFP4Tensor", "FosError",
            "make_config")


def __getattr__(name):
    if name in _EXPORTS:
        from . import fos
        return getattr(fos, name)
    raise AttributeError(name)
