"""Seeded synthetic inputs for the 3-D max-pooling path.

This module only draws random tensors and names the workload shapes.  It
holds none of the pooling arithmetic (no window bounds, no output-size rule,
no reductions), so that the CPU oracle and the HIP path can both take their
inputs from it without sharing any of the method.

Every tensor is drawn on the CPU in float32 from ``torch.Generator`` with a
fixed seed, then rounded to its storage dtype with torch's round-to-nearest-
even conversion, so every consumer sees identical bits.

Distributions:
  ``uniform``  U(-1, 1), as ``rand * 2 - 1``
  ``normal``   N(0, 1)
  ``int4``     integers drawn uniformly from {-4, ..., 4} (exact in every
               dtype; forces many tied window maxima)
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

DTYPES = {
    "float32": torch.float32,
    "float16": torch.float16,
    "bfloat16": torch.bfloat16,
}


def draw(shape, dist: str, dtype: torch.dtype, seed: int) -> torch.Tensor:
    """A CPU tensor of ``shape`` drawn from ``dist`` with ``seed``, rounded
    to ``dtype``."""
    g = torch.Generator().manual_seed(seed)
    shape = tuple(int(v) for v in shape)
    if dist == "uniform":
        t = torch.rand(shape, generator=g, dtype=torch.float32) * 2 - 1
    elif dist == "normal":
        t = torch.randn(shape, generator=g, dtype=torch.float32)
    elif dist == "int4":
        t = torch.randint(-4, 5, shape, generator=g).to(torch.float32)
    else:
        raise ValueError("unknown distribution %r" % dist)
    return t.to(dtype)


@dataclass(frozen=True)
class Workload:
    """One named pooling workload.  Exactly one of ``out`` (adaptive windows,
    output extent per axis) and ``kernel``/``stride`` (fixed windows) is
    set.  ``backward`` says whether a grad_output is drawn for it."""

    name: str
    title: str
    dtype: str
    shape: tuple
    x_dist: str
    backward: bool
    out: tuple | None = None
    kernel: tuple | None = None
    stride: tuple | None = None
    gy_dist: str = "normal"
    x_seed: int = 0
    gy_seed: int = 0

    @property
    def adaptive(self) -> bool:
        return self.out is not None

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    def make_x(self) -> torch.Tensor:
        return draw(self.shape, self.x_dist, self.torch_dtype, self.x_seed)

    def make_gy(self, out_shape) -> torch.Tensor:
        """grad_output of the given (N, C, OD, OH, OW) shape."""
        return draw(out_shape, self.gy_dist, self.torch_dtype, self.gy_seed)


WORKLOADS = (
    Workload("adaptive_f32_divisible",
             "adaptive fwd+bwd, float32 (2,3,8,8,8) -> (4,4,4), windows tile the input",
             "float32", (2, 3, 8, 8, 8), "uniform", True, out=(4, 4, 4),
             x_seed=1001, gy_seed=2001),
    Workload("adaptive_bf16_ties",
             "adaptive fwd+bwd, bfloat16 (4,16,10,10,10) integers in [-4,4] -> (8,8,8), overlapping",
             "bfloat16", (4, 16, 10, 10, 10), "int4", True, out=(8, 8, 8),
             x_seed=1002, gy_seed=2002),
    Workload("fixed_bf16_k2s2",
             "fixed fwd only, bfloat16 (16,64,16,112,112), kernel 2 stride 2",
             "bfloat16", (16, 64, 16, 112, 112), "normal", False,
             kernel=(2, 2, 2), stride=(2, 2, 2), x_seed=1003, gy_seed=2003),
    Workload("fixed_f16_k3s2",
             "fixed fwd+bwd, float16 (8,128,32,56,56), kernel 3 stride 2, overlapping",
             "float16", (8, 128, 32, 56, 56), "normal", True,
             kernel=(3, 3, 3), stride=(2, 2, 2), x_seed=1004, gy_seed=2004),
    Workload("adaptive_f32_large",
             "adaptive fwd+bwd, float32 (32,256,16,32,32) -> (5,7,7), overlapping",
             "float32", (32, 256, 16, 32, 32), "uniform", True, out=(5, 7, 7),
             x_seed=1005, gy_seed=2005),
)

BY_NAME = {w.name: w for w in WORKLOADS}


# The input shapes and dtypes of the latency table on the PR #308 page
# ("[KernelGen][MThreads] Add adaptive_max_pool3d_backward Moore Threads
# specialized operator", Performance).  The page prints no output_size;
# callers pair each shape with output sizes of their own.
PR308_SHAPES = tuple((dt, shape) for dt in ("float16", "float32", "bfloat16")
                     for shape in ((1, 1, 4, 4, 4), (2, 3, 8, 8, 8), (1, 1, 16, 16, 16),
                                   (2, 8, 4, 4, 4)))
