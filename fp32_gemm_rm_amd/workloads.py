"""Seeded synthetic inputs for row-major SGEMM.

This module only draws and lays out input buffers; it holds none of the
operation's arithmetic, so both the GPU path's tests and the CPU oracle can
consume the same arrays.

Every buffer is a flat float32 host array holding ``rows * ld`` elements, with
the logical matrix in the first ``cols`` entries of each row.  Padding between
the logical width and the leading dimension is NaN for A and B (so any read of
it poisons the result) and a fixed finite sentinel for C (so any write to it
is visible).

Draw order is fixed: A (M x K), then B (K x N), then the initial C (M x N)
when it is random, all from one CPU ``torch.Generator`` seeded per workload.
Uniform[-1, 1) is ``2*rand - 1`` (exact in float32: rand yields multiples of
2^-24, so the result is a multiple of 2^-23); normal is ``randn``.  The pages
fill their matrices with ``rand()/RAND_MAX`` and do not seed it
(m.lqnn.cn/news/94381 section 1.3; mlqm.cn/news/1180856 section 5).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

#: Finite sentinel written into C's padding columns; compared bit for bit.
C_PAD_SENTINEL = np.float32(-12345.6789)


@dataclass(frozen=True)
class GemmWorkload:
    """One SGEMM problem: sizes, leading dimensions, scalars and input recipe."""

    name: str
    M: int
    N: int
    K: int
    lda: int
    ldb: int
    ldc: int
    dist: str  # "uniform" (U[-1,1)) or "normal" (N(0,1))
    seed: int
    alpha: float
    beta: float
    c_init: str  # "zeros" or "random" (same distribution as A and B)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


#: The five workloads, smallest first.  4096^3 is the headline benchmark.
WORKLOADS = (
    GemmWorkload("sgemm_256", 256, 256, 256, 256, 256, 256, "uniform", 0, 1.0, 0.0, "zeros"),
    GemmWorkload("sgemm_1024", 1024, 1024, 1024, 1024, 1024, 1024, "uniform", 1, 1.0, 0.0, "zeros"),
    GemmWorkload("sgemm_ragged_1000x1030x999", 1000, 1030, 999, 1008, 1040, 1040, "uniform", 2,
                 1.5, -0.5, "random"),
    GemmWorkload("sgemm_4096", 4096, 4096, 4096, 4096, 4096, 4096, "uniform", 3, 1.0, 0.0, "zeros"),
    GemmWorkload("sgemm_8192", 8192, 8192, 8192, 8192, 8192, 8192, "normal", 4, 1.0, 1.0, "random"),
)
WORKLOAD_BY_NAME = {w.name: w for w in WORKLOADS}
HEADLINE = WORKLOAD_BY_NAME["sgemm_4096"]


def _draw(gen: torch.Generator, rows: int, cols: int, dist: str) -> np.ndarray:
    if dist == "uniform":
        t = torch.rand(rows, cols, generator=gen, dtype=torch.float32) * 2.0 - 1.0
    elif dist == "normal":
        t = torch.randn(rows, cols, generator=gen, dtype=torch.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return t.numpy()


def pad_rows(mat: np.ndarray, ld: int, fill) -> np.ndarray:
    """Lay ``mat`` (rows x cols) into a flat ``rows*ld`` buffer, padding with ``fill``."""
    rows, cols = mat.shape
    if ld < cols:
        raise ValueError(f"leading dimension {ld} < width {cols}")
    buf = np.full((rows, ld), fill, dtype=np.float32)
    buf[:, :cols] = mat
    return buf.reshape(-1)


def make_inputs(M, N, K, lda, ldb, ldc, dist="uniform", seed=0, c_init="zeros"):
    """Return flat float32 buffers (A, B, C) for one problem, padded as described above."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    a = _draw(gen, M, K, dist)
    b = _draw(gen, K, N, dist)
    if c_init == "random":
        c = _draw(gen, M, N, dist)
    elif c_init == "zeros":
        c = np.zeros((M, N), dtype=np.float32)
    elif c_init == "nan":
        c = np.full((M, N), np.nan, dtype=np.float32)
    else:
        raise ValueError(f"unknown C initialisation {c_init!r}")
    return pad_rows(a, lda, np.nan), pad_rows(b, ldb, np.nan), pad_rows(c, ldc, C_PAD_SENTINEL)


def workload_inputs(w: GemmWorkload):
    """Buffers (A, B, C) of a named workload."""
    return make_inputs(w.M, w.N, w.K, w.lda, w.ldb, w.ldc, w.dist, w.seed, w.c_init)


@dataclass(frozen=True)
class BatchedWorkload:
    """A strided batch of equal-shape SGEMMs (contiguous matrices, stride = matrix size)."""

    name: str
    batch: int
    M: int
    N: int
    K: int
    dist: str
    seed: int
    alpha: float
    beta: float

    @property
    def flops(self) -> int:
        return 2 * self.batch * self.M * self.N * self.K


#: Batched workload of "GPU-accelerated matrix computation ..." section 4.2: 1024 products
#: of 64 x 64 matrices in one call (batchCount = 1024; strides M*K, K*N, M*N).
BATCHED_WORKLOADS = (
    BatchedWorkload("sgemm_batched_1024x64", 1024, 64, 64, 64, "uniform", 5, 1.0, 0.0),
)
BATCHED_BY_NAME = {w.name: w for w in BATCHED_WORKLOADS}


def make_batched_inputs(batch, M, N, K, lda, ldb, ldc, sA, sB, sC, dist="uniform", seed=0, c_init="zeros"):
    """Flat buffers (A, B, C) of a strided batch.  Entry b is drawn as make_inputs would draw it
    (A, B, then C) from one generator, in batch order; everything outside the entries' logical
    windows (row padding and the gaps between entries) is NaN for A and B and the C sentinel for C.
    A stride of 0 shares one matrix between all entries (drawn once)."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    nA = max((batch - 1) * sA + (M - 1) * lda + K, M * lda) if batch else 0
    nB = max((batch - 1) * sB + (K - 1) * ldb + N, K * ldb) if batch else 0
    nC = max((batch - 1) * sC + (M - 1) * ldc + N, M * ldc) if batch else 0
    A = np.full(nA, np.nan, np.float32)
    B = np.full(nB, np.nan, np.float32)
    C = np.full(nC, C_PAD_SENTINEL, np.float32)
    for b in range(batch):
        a = _draw(gen, M, K, dist)
        bb = _draw(gen, K, N, dist)
        if c_init == "random":
            c = _draw(gen, M, N, dist)
        elif c_init == "zeros":
            c = np.zeros((M, N), np.float32)
        else:
            c = np.full((M, N), np.nan, np.float32)
        if b == 0 or sA:
            _put(A, b * sA, a, lda)
        if b == 0 or sB:
            _put(B, b * sB, bb, ldb)
        _put(C, b * sC, c, ldc)
    return A, B, C


def _put(buf: np.ndarray, offset: int, mat: np.ndarray, ld: int) -> None:
    """Write mat's rows into the flat buffer at offset, row i at offset + i*ld."""
    rows, cols = mat.shape
    if rows == 0 or cols == 0:
        return
    if offset + rows * ld <= buf.size:
        buf[offset: offset + rows * ld].reshape(rows, ld)[:, :cols] = mat
    else:  # the last entry's last row may end at its logical width
        for i in range(rows):
            buf[offset + i * ld: offset + i * ld + cols] = mat[i]


def integer_matrix(rows: int, cols: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Integer-valued float32 matrix with entries drawn uniformly from [lo, hi]."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    t = torch.randint(lo, hi + 1, (rows, cols), generator=gen, dtype=torch.int64)
    return t.numpy().astype(np.float32)
