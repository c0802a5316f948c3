"""Seeded synthetic inputs for the GEMM workloads.

This module only draws numbers and lays them out in memory.  It holds none of
the GEMM arithmetic, so both the CPU oracle's tests and the GPU library's
tests and benchmark can use it without sharing any of the method.

Conventions
-----------
* Generator: ``numpy.random.Generator(PCG64(seed))``.
* fp32 U[-1,1): ``2*rng.random(n, dtype=float32) - 1`` evaluated in float32.
  ``rng.random`` returns multiples of 2**-24 in [0,1), so the result is an
  exact float32 value in [-1, 1).
* fp32 N(0,1): ``rng.standard_normal(n, dtype=float32)``.
* fp64 U[-1,1): ``2*rng.random(n) - 1`` in float64.
* Draw order: A, then B, then C (only when the workload makes C random).
  Each matrix's logical elements are drawn in storage order: column by column
  for column-major storage, row by row for row-major storage.
* Padding (ld beyond the logical extent) is filled with a caller-chosen value:
  NaN by default for A and B, so that any read of padding poisons the result,
  and a bit-pattern sentinel for C, so that any write to padding shows.

The workloads are the dense square and ragged problems the pages measure
(square N = 2048 as on the vectorized double-buffer page, N <= 512 for the
verify step), plus a row-major fp64 case in the lecture's lda/ldb/ldc form.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# A quiet-NaN float32 with a recognisable payload, used for C padding.
C_SENTINEL_F32 = np.frombuffer(np.uint32(0x7FC0BEEF).tobytes(), dtype=np.float32)[0]
C_SENTINEL_F64 = np.frombuffer(np.uint64(0x7FF8DEADBEEF0001).tobytes(), dtype=np.float64)[0]


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def draw(rng: np.random.Generator, count: int, dist: str, dtype) -> np.ndarray:
    """``count`` values from ``dist`` ('u' = U[-1,1), 'n' = N(0,1), 'i2' =
    integers in {-2..2}, 'ones') in ``dtype``."""
    dtype = np.dtype(dtype)
    if dist == "u":
        if dtype == np.float32:
            x = rng.random(count, dtype=np.float32)
            return (np.float32(2.0) * x - np.float32(1.0)).astype(np.float32)
        return 2.0 * rng.random(count) - 1.0
    if dist == "n":
        return rng.standard_normal(count, dtype=dtype.type)
    if dist == "i2":
        return rng.integers(-2, 3, size=count).astype(dtype)
    if dist == "ones":
        return np.ones(count, dtype=dtype)
    raise ValueError("unknown distribution %r" % dist)


def colmajor(values: np.ndarray, rows: int, cols: int, ld: int, pad) -> np.ndarray:
    """Place ``values`` (rows*cols, column by column) into ld*cols storage."""
    assert ld >= max(1, rows)
    buf = np.full(ld * cols, pad, dtype=values.dtype)
    if rows and cols:
        view = buf.reshape(cols, ld)
        view[:, :rows] = values.reshape(cols, rows)
    return buf


def rowmajor(values: np.ndarray, rows: int, cols: int, ld: int, pad) -> np.ndarray:
    """Place ``values`` (rows*cols, row by row) into rows*ld storage."""
    assert ld >= max(1, cols)
    buf = np.full(ld * rows, pad, dtype=values.dtype)
    if rows and cols:
        view = buf.reshape(rows, ld)
        view[:, :cols] = values.reshape(rows, cols)
    return buf


def logical_colmajor(buf: np.ndarray, rows: int, cols: int, ld: int) -> np.ndarray:
    """(rows, cols) view of the logical block of column-major storage."""
    if rows == 0 or cols == 0:
        return np.zeros((rows, cols), dtype=buf.dtype)
    return buf[: ld * cols].reshape(cols, ld)[:, :rows].T


def logical_rowmajor(buf: np.ndarray, rows: int, cols: int, ld: int) -> np.ndarray:
    if rows == 0 or cols == 0:
        return np.zeros((rows, cols), dtype=buf.dtype)
    return buf[: ld * rows].reshape(rows, ld)[:, :cols]


@dataclasses.dataclass
class Problem:
    """One GEMM problem in storage form (column-major unless ``rowmajor``)."""
    name: str
    dtype: type
    m: int
    n: int
    k: int
    lda: int
    ldb: int
    ldc: int
    alpha: float
    beta: float
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    rowmajor: bool = False   # True: lecture form N1=m, N2=k, N3=n, row-major

    @property
    def flops(self) -> float:
        return 2.0 * self.m * self.n * self.k


def make_colmajor_problem(name, dtype, m, n, k, lda, ldb, ldc, alpha, beta, seed,
                          dist="u", c_dist: Optional[str] = None, c_zero=False,
                          ab_pad=np.nan) -> Problem:
    """Draw A (m x k), B (k x n) and C (m x n) column-major.

    ``c_dist`` None means C is not drawn: it is zero-initialised when
    ``c_zero`` and otherwise filled with NaN (a beta == 0 call must not read
    it).  Padding of C is the sentinel either way.
    """
    dtype = np.dtype(dtype).type
    rng = rng_for(seed)
    sent = C_SENTINEL_F32 if dtype == np.float32 else C_SENTINEL_F64
    A = colmajor(draw(rng, m * k, dist, dtype), m, k, lda, ab_pad)
    B = colmajor(draw(rng, k * n, dist, dtype), k, n, ldb, ab_pad)
    if c_dist is not None:
        cv = draw(rng, m * n, c_dist, dtype)
    elif c_zero:
        cv = np.zeros(m * n, dtype=dtype)
    else:
        cv = np.full(m * n, np.nan, dtype=dtype)
    C = colmajor(cv, m, n, ldc, sent)
    return Problem(name, dtype, m, n, k, lda, ldb, ldc, alpha, beta, A, B, C)


def make_rowmajor_problem(name, N1, N2, N3, lda, ldb, ldc, alpha, beta, seed,
                          dist="u", c_dist="u", ab_pad=np.nan) -> Problem:
    """Lecture-form fp64 problem: A N1 x N2, B N2 x N3, C N1 x N3, row-major."""
    rng = rng_for(seed)
    A = rowmajor(draw(rng, N1 * N2, dist, np.float64), N1, N2, lda, ab_pad)
    B = rowmajor(draw(rng, N2 * N3, dist, np.float64), N2, N3, ldb, ab_pad)
    if c_dist is not None:
        cv = draw(rng, N1 * N3, c_dist, np.float64)
    else:
        cv = np.full(N1 * N3, np.nan)
    C = rowmajor(cv, N1, N3, ldc, C_SENTINEL_F64)
    return Problem(name, np.float64, N1, N3, N2, lda, ldb, ldc, alpha, beta, A, B, C,
                   rowmajor=True)


# ------------------------------------------------------------------ workloads
#
# The five workload families, by what they are:
#   sgemm_128        square 128^3, U[-1,1) seed 0, alpha=1, beta=0, C zeroed
#   sgemm_2048       square 2048^3, U[-1,1) seed 1, alpha=1, beta=0
#   sgemm_sweep_N    square N^3 for N in 512..8192, A,B,C U[-1,1) seed 2,
#                    alpha=1.5, beta=0.5
#   sgemm_ragged     4097 x 3001 x 1023, ld = dim + 16, A,B,C N(0,1) seed 3,
#                    alpha=0.75, beta=-1.25
#   dgemm_rowmajor   fp64 row-major 4096^3 with ld 4104, A,B,C U[-1,1) seed 4,
#                    alpha=1, beta=1 (the lecture's C += A*B)
#   sgemm_shard_8192_g8
#                    one GPU's share when sgemm_sweep_8192 is split by columns
#                    of C over 8 GPUs: the last 1024 columns of B and C (the
#                    same values, ld 8192), all of A: 8192 x 1024 x 8192

SWEEP_SIZES = (512, 1024, 2048, 4096, 8192)


def workload(name: str, dist_override: Optional[str] = None) -> Problem:
    """Build a named workload.  ``dist_override`` replaces every drawn
    distribution (e.g. 'i2' for exact-integer variants of the same shape)."""
    d = lambda x: dist_override if dist_override is not None else x  # noqa: E731
    if name == "sgemm_128":
        return make_colmajor_problem(name, np.float32, 128, 128, 128, 128, 128, 128,
                                     1.0, 0.0, 0, dist=d("u"), c_zero=True)
    if name == "sgemm_2048":
        return make_colmajor_problem(name, np.float32, 2048, 2048, 2048, 2048, 2048,
                                     2048, 1.0, 0.0, 1, dist=d("u"), c_zero=True)
    if name.startswith("sgemm_sweep_"):
        N = int(name.rsplit("_", 1)[1])
        return make_colmajor_problem(name, np.float32, N, N, N, N, N, N, 1.5, 0.5, 2,
                                     dist=d("u"), c_dist=d("u"))
    if name == "sgemm_ragged":
        M, N, K = 4097, 3001, 1023
        return make_colmajor_problem(name, np.float32, M, N, K, M + 16, K + 16, M + 16,
                                     0.75, -1.25, 3, dist=d("n"), c_dist=d("n"))
    if name == "dgemm_rowmajor":
        n = 4096
        return make_rowmajor_problem(name, n, n, n, n + 8, n + 8, n + 8, 1.0, 1.0, 4,
                                     dist=d("u"), c_dist=d("u"))
    if name == "sgemm_shard_8192_g8":
        full = workload("sgemm_sweep_8192", dist_override)
        shards, n = 8, full.n // 8
        j0 = (shards - 1) * n
        return Problem(name, np.float32, full.m, n, full.k, full.lda, full.ldb, full.ldc,
                       full.alpha, full.beta, full.A, full.B[j0 * full.ldb:(j0 + n) * full.ldb],
                       full.C[j0 * full.ldc:(j0 + n) * full.ldc])
    raise KeyError(name)


SHARD_COLUMN0 = {"sgemm_shard_8192_g8": 7 * 1024}   # first column of the shard

WORKLOADS = (["sgemm_128", "sgemm_2048"]
             + ["sgemm_sweep_%d" % n for n in SWEEP_SIZES]
             + ["sgemm_ragged", "dgemm_rowmajor", "sgemm_shard_8192_g8"])
