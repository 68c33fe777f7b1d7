"""Seeded synthetic inputs for C = alpha*A.B + beta*C0 -- shared by tests and bench.

This module holds no arithmetic of the method: it only draws random numbers,
rounds them to the storage dtype and places them in (possibly padded) row-major
buffers.  Both the GPU path's tests and the CPU oracle take their inputs from
here; nothing here imports either of them.

Recipe (the pages print no workload; these are the five problem shapes the
build is measured on):
  * one ``torch.Generator('cpu')`` per problem, seeded (default 0);
  * draws in the order A, B, C0, as float32: U[-1, 1) is ``rand*2-1``,
    N(0, s) is ``randn*s``;
  * A and B are rounded to their storage dtype with round-to-nearest-even
    (``torch.Tensor.to``); the oracle and the GPU both consume the rounded values;
  * leading-dimension padding (lda - K columns of A, ldb - N of B) is filled
    with NaN, so a kernel that reads past an extent is caught;
  * C0 exists only when beta != 0; it is float32 with ldc padding NaN.
Storage: bf16/f16 as uint16 bit patterns, f32 as float32, all flat and C-contiguous.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

NAN_BITS = {"bf16": 0x7FC0, "f16": 0x7E00}
TORCH_DTYPE = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@dataclass
class Problem:
    name: str
    dtype: str                  # 'f32' | 'bf16' | 'f16' (A and B); C is always float32
    M: int
    N: int
    K: int
    batch: int = 1
    lda: Optional[int] = None
    ldb: Optional[int] = None
    ldc: Optional[int] = None
    strideA: Optional[int] = None
    strideB: Optional[int] = None
    strideC: Optional[int] = None
    alpha: float = 1.0
    beta: float = 0.0
    dist: str = "uniform"       # 'uniform' (U[-1,1)) | 'normal' (N(0, sigma)) | 'int' (integers in [-ilim, ilim])
    sigma: float = 1.0
    ilim: int = 2
    c0_ilim: int = 1024
    seed: int = 0
    note: str = ""
    A: Optional[np.ndarray] = field(default=None, repr=False)
    B: Optional[np.ndarray] = field(default=None, repr=False)
    C0: Optional[np.ndarray] = field(default=None, repr=False)

    def __post_init__(self):
        self.lda = self.K if self.lda is None else self.lda
        self.ldb = self.N if self.ldb is None else self.ldb
        self.ldc = self.N if self.ldc is None else self.ldc
        self.lda = max(self.lda, 1)
        self.ldb = max(self.ldb, 1)
        self.ldc = max(self.ldc, 1)
        if self.strideA is None:
            self.strideA = self.M * self.lda
        if self.strideB is None:
            self.strideB = self.K * self.ldb
        if self.strideC is None:
            self.strideC = self.M * self.ldc

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.batch

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def sizeA(self) -> int:
        return max(0, (self.batch - 1) * self.strideA + self.M * self.lda) if self.batch and self.M else 0

    def sizeB(self) -> int:
        return max(0, (self.batch - 1) * self.strideB + self.K * self.ldb) if self.batch and self.K else 0

    def sizeC(self) -> int:
        return max(0, (self.batch - 1) * self.strideC + self.M * self.ldc) if self.batch and self.M else 0

    def compulsory_bytes(self) -> int:
        """A and B read once, C written once (and read once when beta != 0)."""
        e = self.elem_bytes
        c = 4 * self.batch * self.M * self.N
        return e * self.batch * (self.M * self.K + self.K * self.N) + c * (2 if self.beta != 0 else 1)


# The five problem shapes (the pages give none of their own).
CONFIGS = {
    "c1_f32_67x45x53": Problem("c1_f32_67x45x53", "f32", 67, 45, 53, dist="uniform",
                               note="fp32, non-tile-multiple, contiguous, beta=0"),
    "c2_bf16_8192": Problem("c2_bf16_8192", "bf16", 8192, 8192, 8192, dist="normal", sigma=1.0,
                            note="bf16 in / fp32 out, square 8192^3, beta=0"),
    "c3_bf16_ragged": Problem("c3_bf16_ragged", "bf16", 8191, 8193, 8190, lda=8190 + 3, ldb=8193 + 5,
                              alpha=1.5, beta=0.5, dist="uniform",
                              note="ragged extents, padded strides, alpha=1.5 beta=0.5, C0 ~ N(0,1)"),
    "c4_f16_batched": Problem("c4_f16_batched", "f16", 257, 129, 1000, batch=512, dist="normal", sigma=0.1,
                              note="512 packed fp16 GEMMs, HBM-bound"),
    "c5_bf16_deepk": Problem("c5_bf16_deepk", "bf16", 512, 512, 131072, dist="uniform",
                             note="K-dominant, 512x512x131072"),
}


def _draw(g: torch.Generator, shape, p: Problem) -> torch.Tensor:
    n = int(np.prod(shape)) if len(shape) else 1
    if n == 0:
        return torch.empty(shape, dtype=torch.float32)
    if p.dist == "uniform":
        return torch.rand(shape, generator=g, dtype=torch.float32) * 2 - 1
    if p.dist == "normal":
        return torch.randn(shape, generator=g, dtype=torch.float32) * p.sigma
    if p.dist == "int":
        return torch.randint(-p.ilim, p.ilim + 1, shape, generator=g).to(torch.float32)
    raise ValueError(p.dist)


def _to_storage(t: torch.Tensor, dtype: str) -> np.ndarray:
    r = t.to(TORCH_DTYPE[dtype]).contiguous()
    if dtype == "f32":
        return r.numpy()
    return r.view(torch.int16).numpy().view(np.uint16)


def _place(vals: np.ndarray, batch, rows, cols, ld, stride, dtype) -> np.ndarray:
    """Put (batch, rows, cols) values into a flat padded buffer, NaN elsewhere."""
    size = (batch - 1) * stride + rows * ld if batch and rows else 0
    if dtype == "f32":
        buf = np.full(size, np.nan, dtype=np.float32)
    else:
        buf = np.full(size, NAN_BITS[dtype], dtype=np.uint16)
    if size == 0 or cols == 0:
        return buf
    if ld == cols and stride == rows * ld:
        buf[:] = vals.reshape(-1)
        return buf
    for b in range(batch):
        view = buf[b * stride: b * stride + rows * ld].reshape(rows, ld)
        view[:, :cols] = vals[b]
    return buf


def materialize(p: Problem) -> Problem:
    """Return a copy of p with A, B (and C0 if beta != 0) drawn from its seed."""
    g = torch.Generator(device="cpu")
    g.manual_seed(p.seed)
    a = _to_storage(_draw(g, (p.batch, p.M, p.K), p), p.dtype)
    b = _to_storage(_draw(g, (p.batch, p.K, p.N), p), p.dtype)
    A = _place(a.reshape(p.batch, p.M, p.K), p.batch, p.M, p.K, p.lda, p.strideA, p.dtype)
    B = _place(b.reshape(p.batch, p.K, p.N), p.batch, p.K, p.N, p.ldb, p.strideB, p.dtype)
    C0 = None
    if p.beta != 0.0:
        if p.dist == "int":
            c = torch.randint(-p.c0_ilim, p.c0_ilim + 1, (p.batch, p.M, p.N), generator=g).to(torch.float32)
        else:
            c = torch.randn((p.batch, p.M, p.N), generator=g, dtype=torch.float32)
        C0 = _place(c.numpy(), p.batch, p.M, p.N, p.ldc, p.strideC, "f32")
    return replace(p, A=A, B=B, C0=C0)


# Further shapes the benchmark can time (not among the five: the large fp32 problem the fp32
# ring tiles are measured on).
EXTRA = {
    "f32_8192": Problem("f32_8192", "f32", 8192, 8192, 8192, dist="uniform",
                        note="fp32 in / fp32 out, square 8192^3, beta=0 (fp32 ring tile)"),
}


def config(name: str, seed: int = 0) -> Problem:
    return materialize(replace(CONFIGS[name] if name in CONFIGS else EXTRA[name], seed=seed))


def custom(dtype, M, N, K, batch=1, lda_pad=0, ldb_pad=0, ldc_pad=0, alpha=1.0, beta=0.0,
           dist="uniform", sigma=1.0, seed=0, packed_batch=True, name="custom", **kw) -> Problem:
    """A problem with the same recipe at other extents (lda = K + lda_pad, ...)."""
    p = Problem(name, dtype, M, N, K, batch=batch, lda=K + lda_pad, ldb=N + ldb_pad,
                ldc=N + ldc_pad, alpha=alpha, beta=beta, dist=dist, sigma=sigma, seed=seed, **kw)
    return materialize(p)


def sample_points(p: Problem, n: int, seed: int = 1) -> np.ndarray:
    """(b, i, j) output coordinates: the whole last row and last column of every batch entry
    (of the first and last when that would exceed 300k points), where thin fringe strips and
    fringe tiles end; corners and middles; then n random points."""
    rng = np.random.default_rng(seed)
    fixed = []
    for b in sorted({0, p.batch - 1}):
        for i in sorted({0, p.M - 1, max(0, p.M // 2)}):
            for j in sorted({0, p.N - 1, max(0, p.N // 2)}):
                fixed.append((b, i, j))
    edge_entries = range(p.batch) if p.batch * (p.M + p.N) <= 300000 else sorted({0, p.batch - 1})
    for b in edge_entries:
        fixed += [(b, p.M - 1, j) for j in range(p.N)]
        fixed += [(b, i, p.N - 1) for i in range(p.M)]
    fixed = sorted(set(fixed))
    rest = n
    rnd = np.stack([rng.integers(0, p.batch, rest), rng.integers(0, p.M, rest),
                    rng.integers(0, p.N, rest)], axis=1) if rest else np.zeros((0, 3), np.int64)
    pts = np.concatenate([np.array(fixed, dtype=np.int64).reshape(-1, 3), rnd.astype(np.int64)])
    return pts
