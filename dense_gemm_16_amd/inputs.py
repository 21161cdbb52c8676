"""Seeded synthetic inputs for the dense matrix product.

This module holds no part of the product's arithmetic: it only draws and
rounds input matrices on the CPU with torch, so that the GPU library and the
CPU oracle receive the very same stored values.  The oracle never imports the
GPU library, and this module imports neither.

Recipes (one CPU ``torch.Generator`` per draw, seeded; A is drawn before B):

* ``uniform``: binary32 values ``rand * 2 - 1`` in [-1, 1), then rounded to
  the input type with round-to-nearest-even (torch ``.to``), as the
  ``__float2half`` conversion on page "04-wmma-matmul.cu" does.  A value may
  round to exactly 1.0 in FP16/BF16.
* ``normal``: binary32 standard normal draws, rounded the same way.
* ``int``: integers uniform in [lo, hi] inclusive, stored exactly in the type.
* ``p3``: the exact small-integer pattern of page "matmul_registers.cu"
  (``fillInputs``): a = ((row + 2 col) mod 7) - 3, b = ((3 row + col) mod 5) - 2,
  extended to rectangular shapes with the same row/col formula.
* ``p1``: the modular pattern of page "04-wmma-matmul.cu" in flat index i:
  a = ((7 i + 1) mod 13)/13 - 0.5, b = ((5 i + 3) mod 11)/11 - 0.5.

INT8 (``i8``) takes integers only: ``uniform`` is uniform over -128 .. 127 and
``int`` over [lo, hi]; nothing is rounded.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
                "i8": torch.int8}
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1}
OUT_BYTES = {"f32": 4, "f16": 4, "bf16": 4, "i8": 4}  # C: FP32, or INT32 for INT8


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def draw(shape, dtype: str, dist: str, g: torch.Generator, lo: int = -4, hi: int = 4):
    """One matrix of ``shape`` in storage type ``dtype`` (CPU tensor)."""
    t = TORCH_DTYPES[dtype]
    if dtype == "i8":
        if dist == "zeros":
            return torch.zeros(shape, dtype=torch.int8)
        if dist == "uniform":
            lo, hi = -128, 127
        elif dist != "int":
            raise ValueError(f"INT8 inputs take the uniform, int or zeros distributions, not {dist!r}")
        return torch.randint(lo, hi + 1, shape, generator=g, dtype=torch.int32).to(torch.int8)
    if dist == "uniform":
        x = torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0
    elif dist == "normal":
        x = torch.randn(shape, generator=g, dtype=torch.float32)
    elif dist == "int":
        x = torch.randint(lo, hi + 1, shape, generator=g, dtype=torch.int32).to(torch.float32)
    elif dist == "ones":
        x = torch.ones(shape, dtype=torch.float32)
    elif dist == "zeros":
        x = torch.zeros(shape, dtype=torch.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return x.to(t)


def pair(M: int, N: int, K: int, dtype: str, dist: str, seed: int, lo: int = -4, hi: int = 4):
    """(A, B) with A of M x K and B of K x N, both drawn from one generator, A first."""
    g = _gen(seed)
    if dist == "p3":
        r = torch.arange(M).view(-1, 1)
        c = torch.arange(K).view(1, -1)
        a = (((r + 2 * c) % 7) - 3).to(torch.float32)
        r = torch.arange(K).view(-1, 1)
        c = torch.arange(N).view(1, -1)
        b = (((3 * r + c) % 5) - 2).to(torch.float32)
        return a.to(TORCH_DTYPES[dtype]), b.to(TORCH_DTYPES[dtype])
    if dist == "p1":
        ia = torch.arange(M * K, dtype=torch.int64)
        ib = torch.arange(K * N, dtype=torch.int64)
        a = (((ia * 7 + 1) % 13).to(torch.float32) / 13.0 - 0.5).view(M, K)
        b = (((ib * 5 + 3) % 11).to(torch.float32) / 11.0 - 0.5).view(K, N)
        return a.to(TORCH_DTYPES[dtype]), b.to(TORCH_DTYPES[dtype])
    A = draw((M, K), dtype, dist, g, lo, hi)
    B = draw((K, N), dtype, dist, g, lo, hi)
    return A, B


def with_ld(x: torch.Tensor, ld: int) -> torch.Tensor:
    """A view of ``x`` with row stride ``ld`` >= its width (padding is NaN where representable)."""
    rows, cols = x.shape
    if ld == cols:
        return x
    if ld < cols:
        raise ValueError("ld must be at least the row width")
    buf = torch.full((max(rows, 1), ld), float("nan"), dtype=x.dtype)
    buf[:rows, :cols] = x
    return buf[:rows, :cols]


def to_bits(x: torch.Tensor) -> np.ndarray:
    """The stored encoding as numpy: float32 for FP32, raw uint16 bits for FP16/BF16,
    int8 for INT8."""
    x = x.detach().cpu()
    if x.dtype in (torch.float32, torch.int8):
        return x.numpy()
    return x.view(torch.int16).numpy().view(np.uint16)


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dtype: str
    dist: str
    seed: int
    exact: bool = False

    @property
    def flop(self) -> float:
        return 2.0 * self.M * self.N * self.K

    def compulsory_bytes(self) -> int:
        e = ELEM_BYTES[self.dtype]
        return e * (self.M * self.K + self.K * self.N) + OUT_BYTES[self.dtype] * self.M * self.N

    def make(self):
        return pair(self.M, self.N, self.K, self.dtype, self.dist, self.seed)


# The benchmark workloads: row-major, dense leading dimensions, seeded.
WORKLOADS = {w.name: w for w in [
    Workload("c0-f16-256", 256, 256, 256, "f16", "uniform", 0),
    Workload("c1-f32-1024", 1024, 1024, 1024, "f32", "uniform", 1),
    Workload("c1-f32-1024-int", 1024, 1024, 1024, "f32", "int", 11, exact=True),
    Workload("c2-f16-1024", 1024, 1024, 1024, "f16", "uniform", 2),
    Workload("c3-f16-2048", 2048, 2048, 2048, "f16", "normal", 3),
    Workload("c3-bf16-2048", 2048, 2048, 2048, "bf16", "normal", 13),
    Workload("c3r-f16-2050x2047x2056", 2050, 2047, 2056, "f16", "normal", 23),
    Workload("c4-bf16-8192", 8192, 8192, 8192, "bf16", "normal", 4),
    Workload("c4f-f32-4096", 4096, 4096, 4096, "f32", "uniform", 14),
    # INT8 -> INT32 at the headline size (not one of the measured configurations of the
    # pages; timed as an extra line)
    Workload("i8-8192", 8192, 8192, 8192, "i8", "uniform", 5, exact=True),
    # one GPU's share of the 8192^3 BF16 product split over rows of C across 8 GPUs,
    # and over a 2 x 4 grid of (rows, columns) (timed as extra lines)
    Workload("s8-bf16-1024x8192x8192", 1024, 8192, 8192, "bf16", "normal", 6),
    Workload("s2x4-bf16-4096x2048x8192", 4096, 2048, 8192, "bf16", "normal", 7),
    # a long K on a few tiles of C (summed as slices of K; timed as extra lines)
    Workload("lk-bf16-512x512x65536", 512, 512, 65536, "bf16", "normal", 8),
    Workload("lk-f32-512x512x16384", 512, 512, 16384, "f32", "uniform", 9),
    # INT8 rows of 1000 bytes, off 16-byte boundaries (copied first; an extra line)
    Workload("i8u-1000", 1000, 1000, 1000, "i8", "uniform", 10, exact=True),
    # FP32 rows of 2049 elements, off 16-byte boundaries (copied first; an extra line)
    Workload("f32u-2049", 2049, 2049, 2049, "f32", "uniform", 15),
]}
