"""CPU oracle for C <- alpha*A*B + beta*C -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The pgemm library never does, and this package never
imports the library: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64 accumulation, sequential
sum over the inner index, OpenMP over output columns only).  This module only
builds that file with the host C compiler and marshals numpy arrays into it.

Definitions followed (see the header of ``oracle.c`` for the formulas):
  * column-major, A and B not transposed -- "optimizing-sgemm-on-nvidia-
    turing-gpus", introduction (column-major SGEMM, A and B not transposed);
  * row-major ``matmat`` with lda/ldb/ldc, A N1 x N2, B N2 x N3, C N1 x N3 --
    "HPC - Lecture 13 - MatMat GPU", sections "function matmatgpu1" and
    "Kernel 1: Global Memory Access".

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against exact rational arithmetic, closed forms, the identity, the transpose
identity, linearity and numpy special cases; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
          "-shared", "-fPIC"]


def compile_source(src: str, out: str) -> str:
    """Compile a C source file of the oracle's form into a shared library."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no FP contraction)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    return compile_source(SOURCE, LIB_PATH)


def _span(rows, cols, ld):
    """Elements spanned by a column-major rows x cols matrix with leading dim ld."""
    if rows <= 0 or cols <= 0:
        return 0
    return ld * (cols - 1) + rows


def _ptr(a):
    return None if a is None else a.ctypes.data


def _arr(a, dtype, need):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=dtype).reshape(-1)
    if a.size < need:
        raise ValueError("oracle: buffer holds %d elements, needs %d" % (a.size, need))
    return a


def _idx(I, J, rows, cols):
    I = np.ascontiguousarray(I, dtype=np.int64).reshape(-1)
    J = np.ascontiguousarray(J, dtype=np.int64).reshape(-1)
    if I.shape != J.shape:
        raise ValueError("I and J differ in shape")
    if I.size and (I.min() < 0 or I.max() >= rows or J.min() < 0 or J.max() >= cols):
        raise ValueError("entry index out of range")
    return I, J


class OracleLib:
    """ctypes view of one build of ``oracle.c``."""

    def __init__(self, path: str = LIB_PATH):
        lib = ctypes.CDLL(path)
        vp, i, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        gemm_args = [i, i, i, d, vp, i, vp, i, d, vp, i, vp, i]
        ent_args = [i, i, i, d, vp, i, vp, i, d, vp, i, i, vp, vp, vp]
        for name in ("oracle_gemm_f32", "oracle_gemm_f64"):
            getattr(lib, name).argtypes = gemm_args
            getattr(lib, name).restype = None
        for name in ("oracle_gemm_f32_entries", "oracle_gemm_f64_entries"):
            getattr(lib, name).argtypes = ent_args
            getattr(lib, name).restype = None
        lib.oracle_matmat_rowmajor_f64.argtypes = [i, i, i, vp, vp, vp, i, i, i, d, d, vp]
        lib.oracle_matmat_rowmajor_f64.restype = None
        lib.oracle_matmat_rowmajor_f64_entries.argtypes = [i, i, i, vp, vp, vp, i, i, i,
                                                           d, d, i, vp, vp, vp]
        lib.oracle_matmat_rowmajor_f64_entries.restype = None
        lib.oracle_num_threads.restype = i
        lib.oracle_set_num_threads.argtypes = [i]
        self.lib = lib
        self.path = path

    # -- column-major ------------------------------------------------------
    def gemm(self, m, n, k, alpha, A, lda, B, ldb, beta, C0, ldc, dtype=np.float32):
        """Column-major R = alpha*A*B + beta*C0 in double, as an (m, n) array.

        A, B, C0 are 1-D storage buffers (element (i,j) at [i + j*ld]).  R is
        never rounded to ``dtype``.  A/B are not read when k == 0 or alpha ==
        0; C0 is not read when beta == 0 (pass None there if you like).
        """
        use_ab = k > 0 and alpha != 0
        A = _arr(A, dtype, _span(m, k, lda)) if use_ab else None
        B = _arr(B, dtype, _span(k, n, ldb)) if use_ab else None
        C0 = _arr(C0, dtype, _span(m, n, ldc)) if beta != 0 else None
        R = np.empty((n, m), dtype=np.float64)  # column-major, ldr = m
        if m > 0 and n > 0:
            fn = (self.lib.oracle_gemm_f32 if np.dtype(dtype) == np.float32
                  else self.lib.oracle_gemm_f64)
            fn(m, n, k, float(alpha), _ptr(A), lda, _ptr(B), ldb, float(beta),
               _ptr(C0), ldc, _ptr(R), max(m, 1))
        return R.T

    def gemm_entries(self, m, n, k, alpha, A, lda, B, ldb, beta, C0, ldc, I, J,
                     dtype=np.float32):
        """R(I[t], J[t]) for each t: one sequential dot product per entry."""
        use_ab = k > 0 and alpha != 0
        A = _arr(A, dtype, _span(m, k, lda)) if use_ab else None
        B = _arr(B, dtype, _span(k, n, ldb)) if use_ab else None
        C0 = _arr(C0, dtype, _span(m, n, ldc)) if beta != 0 else None
        I, J = _idx(I, J, m, n)
        out = np.empty(I.size, dtype=np.float64)
        fn = (self.lib.oracle_gemm_f32_entries if np.dtype(dtype) == np.float32
              else self.lib.oracle_gemm_f64_entries)
        fn(m, n, k, float(alpha), _ptr(A), lda, _ptr(B), ldb, float(beta), _ptr(C0),
           ldc, int(I.size), _ptr(I), _ptr(J), _ptr(out))
        return out

    # -- row-major lecture form -------------------------------------------
    def matmat_rowmajor_f64(self, lda, ldb, ldc, A, B, C0, N1, N2, N3,
                            alpha=1.0, beta=1.0):
        """Row-major R (N1 x N3) = alpha*A*B + beta*C0; the lecture has alpha=beta=1."""
        use_ab = N2 > 0 and alpha != 0
        A = _arr(A, np.float64, _span(N2, N1, lda)) if use_ab else None
        B = _arr(B, np.float64, _span(N3, N2, ldb)) if use_ab else None
        C0 = _arr(C0, np.float64, _span(N3, N1, ldc)) if beta != 0 else None
        R = np.empty((N1, N3), dtype=np.float64)
        if N1 > 0 and N3 > 0:
            self.lib.oracle_matmat_rowmajor_f64(lda, ldb, ldc, _ptr(A), _ptr(B), _ptr(C0),
                                                N1, N2, N3, float(alpha), float(beta),
                                                _ptr(R))
        return R

    def matmat_rowmajor_f64_entries(self, lda, ldb, ldc, A, B, C0, N1, N2, N3, I, J,
                                    alpha=1.0, beta=1.0):
        use_ab = N2 > 0 and alpha != 0
        A = _arr(A, np.float64, _span(N2, N1, lda)) if use_ab else None
        B = _arr(B, np.float64, _span(N3, N2, ldb)) if use_ab else None
        C0 = _arr(C0, np.float64, _span(N3, N1, ldc)) if beta != 0 else None
        I, J = _idx(I, J, N1, N3)
        out = np.empty(I.size, dtype=np.float64)
        self.lib.oracle_matmat_rowmajor_f64_entries(
            lda, ldb, ldc, _ptr(A), _ptr(B), _ptr(C0), N1, N2, N3, float(alpha),
            float(beta), int(I.size), _ptr(I), _ptr(J), _ptr(out))
        return out

    # -- threads -----------------------------------------------------------
    def num_threads(self) -> int:
        return self.lib.oracle_num_threads()

    def set_num_threads(self, t: int) -> None:
        self.lib.oracle_set_num_threads(int(t))


_default = None


def default() -> OracleLib:
    """The oracle built from ``oracle.c`` (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build()
        _default = OracleLib(LIB_PATH)
    return _default


def gemm(*args, **kw):
    return default().gemm(*args, **kw)


def gemm_entries(*args, **kw):
    return default().gemm_entries(*args, **kw)


def matmat_rowmajor_f64(*args, **kw):
    return default().matmat_rowmajor_f64(*args, **kw)


def matmat_rowmajor_f64_entries(*args, **kw):
    return default().matmat_rowmajor_f64_entries(*args, **kw)


def num_threads() -> int:
    return default().num_threads()


def set_num_threads(t: int) -> None:
    default().set_num_threads(t)


def timed_gemm(m, n, k, alpha, A, lda, B, ldb, beta, C0, ldc, dtype=np.float32):
    """Run the column-major oracle once; return (R, wall seconds)."""
    o = default()
    t0 = time.perf_counter()
    R = o.gemm(m, n, k, alpha, A, lda, B, ldb, beta, C0, ldc, dtype=dtype)
    return R, time.perf_counter() - t0
