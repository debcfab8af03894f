"""Seeded synthetic inputs shared by the tests, the bench and the CPU oracle's callers.

This module holds no quantization arithmetic: it only draws random tensors with the
shapes and value distributions of the workloads and rounds them to bfloat16.  Both
the HIP path and the oracle receive the same bytes from here.

Workloads (shapes stand in for the projections of an 8B-class model; the pages name
Qwen3-8B on the Four Over Six documentation page, §Four Over Six, whose weights are
not used):

  page_example  4096 fp32 values, N(0,1) from torch.manual_seed(0), every 512th
                value times 20 (Ultralytics glossary "FP4", §How FP4 works, the
                worked example).
  c1            256x256 bf16, same recipe as page_example on 65,536 values: the
                x20 outliers are applied in fp32 before rounding to bf16.
  c2            4096x12288 bf16 weight, N(0, 0.02), 0.1 % of the entries (positions
                from a seeded permutation) times 50.
  c3            8192x4096 bf16 activation, 0.5 * Student-t(nu=3).
  c4a           8192x4096 bf16 gradient, N(0, 1e-3).
  c4b           12288x4096 bf16 weight, N(0, 0.02).
  c5_x, c5_w    qlinear operands: X 8192x4096 Student-t(nu=3), W 12288x4096 N(0, 0.02).
  c5_dy         output gradient of that layer for the backward products: 8192x12288
                N(0, 1e-3) (the gradient recipe of c4a).
"""
from __future__ import annotations

import torch

__all__ = [
    "normal_with_outliers",
    "page_example",
    "make",
    "random_bf16",
    "SHAPES",
]

SHAPES = {
    "c1": (256, 256),
    "c2": (4096, 12288),
    "c3": (8192, 4096),
    "c4a": (8192, 4096),
    "c4b": (12288, 4096),
    "c5_x": (8192, 4096),
    "c5_w": (12288, 4096),
    "c5_dy": (8192, 12288),
}


def normal_with_outliers(shape, seed: int = 0, every: int = 512,
                         factor: float = 20.0) -> torch.Tensor:
    """fp32 N(0,1) values from torch's global generator seeded with ``seed``, with
    every ``every``-th value of the flat tensor multiplied by ``factor`` (in fp32).
    The worked example of the Ultralytics glossary page "FP4" (§How FP4 works) draws
    its tensor this way with seed 0, every 512th value, factor 20."""
    torch.manual_seed(seed)
    x = torch.randn(*shape)
    x.view(-1)[::every] *= factor
    return x


def page_example() -> torch.Tensor:
    """The worked example's input: 4096 fp32 values of ``normal_with_outliers``."""
    return normal_with_outliers((4096,))


def _student_t(shape, seed: int, scale: float) -> torch.Tensor:
    torch.manual_seed(seed)
    d = torch.distributions.StudentT(torch.tensor(3.0))
    return scale * d.sample(shape)


def make(name: str) -> torch.Tensor:
    """Return the named workload as a contiguous CPU bfloat16 tensor."""
    shape = SHAPES[name]
    if name == "c1":
        x = normal_with_outliers(shape)
    elif name == "c2":
        g = torch.Generator().manual_seed(2)
        x = 0.02 * torch.randn(*shape, generator=g)
        n_out = round(0.001 * x.numel())
        idx = torch.randperm(x.numel(), generator=g)[:n_out]
        x.view(-1)[idx] *= 50
    elif name == "c3":
        x = _student_t(shape, 3, 0.5)
    elif name == "c4a":
        g = torch.Generator().manual_seed(4)
        x = 1e-3 * torch.randn(*shape, generator=g)
    elif name == "c4b":
        g = torch.Generator().manual_seed(5)
        x = 0.02 * torch.randn(*shape, generator=g)
    elif name == "c5_x":
        x = _student_t(shape, 6, 1.0)
    elif name == "c5_w":
        g = torch.Generator().manual_seed(7)
        x = 0.02 * torch.randn(*shape, generator=g)
    elif name == "c5_dy":
        g = torch.Generator().manual_seed(8)
        x = 1e-3 * torch.randn(*shape, generator=g)
    else:  # pragma: no cover - guarded by SHAPES lookup
        raise KeyError(name)
    return x.to(torch.bfloat16).contiguous()


def random_bf16(rows: int, cols: int, seed: int, dist: str = "normal",
                scale: float = 1.0, outlier_every: int = 0,
                outlier_mult: float = 20.0) -> torch.Tensor:
    """Small seeded bf16 tensors for parity cases.

    dist: "normal" | "student_t" | "uniform" | "zeros".
    outlier_every > 0 multiplies every n-th flat value by outlier_mult (in fp32,
    before the bf16 rounding).
    """
    g = torch.Generator().manual_seed(seed)
    if dist == "normal":
        x = torch.randn(rows, cols, generator=g)
    elif dist == "uniform":
        x = torch.rand(rows, cols, generator=g) * 2 - 1
    elif dist == "student_t":
        # Student-t(3) as N / sqrt(chi2_3 / 3), drawn from the same generator.
        z = torch.randn(rows, cols, generator=g)
        c = (torch.randn(rows, cols, 3, generator=g) ** 2).sum(-1)
        x = z / torch.sqrt(c / 3.0)
    elif dist == "zeros":
        x = torch.zeros(rows, cols)
    else:
        raise ValueError(dist)
    x = x * scale
    if outlier_every > 0 and x.numel() > 0:
        x.view(-1)[::outlier_every] *= outlier_mult
    return x.to(torch.bfloat16).contiguous()
