"""Pins for the CPU oracle: checks that fix its arithmetic from outside it.

Each ``pin_*`` function takes one build of the oracle (``oracle.OracleLib``)
and raises AssertionError if that build disagrees with something the pages or
the mathematics fix independently of the oracle's own code:

  * hand-worked examples computed on paper (``tests/golden``),
  * exact rational arithmetic (``fractions.Fraction``) on tiny inputs with the
    rigorous bound of a double-precision dot product,
  * the identity matrix, closed-form sums, the transpose identity, the
    row-major / column-major operand-swap identity, linearity in alpha and
    beta, and numpy's own float64 routines for the special cases outer
    product, dot product and matrix-vector product.

The same functions run against deliberately broken builds of ``oracle.c`` in
``test_oracle_pins.py`` to show that each plausible mistake trips a pin.
"""
from __future__ import annotations

import os
import sys
from fractions import Fraction

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import gemm_inputs as gi  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U64 = Fraction(1, 2 ** 53)


def gamma(nn: int) -> Fraction:
    """Higham's gamma_n = n*u / (1 - n*u) for double precision."""
    return nn * U64 / (1 - nn * U64)


def read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = rest
    return vals


def _nums(tokens, dtype):
    return np.array([float(t) for t in tokens], dtype=dtype)


# ----------------------------------------------------------------- golden
def pin_golden(o):
    g = read_golden("handworked_colmajor.txt")
    iv = {k: int(g[k][0]) for k in ("m", "n", "k", "lda", "ldb", "ldc")}
    for dtype in (np.float32, np.float64):
        R = o.gemm(iv["m"], iv["n"], iv["k"], float(g["alpha"][0]),
                   _nums(g["A"], dtype), iv["lda"], _nums(g["B"], dtype), iv["ldb"],
                   float(g["beta"][0]), _nums(g["C0"], dtype), iv["ldc"], dtype=dtype)
        want = _nums(g["R"], np.float64).reshape(iv["n"], iv["m"]).T
        assert np.array_equal(R, want), (dtype, R, want)
        # the entries form on every element
        I, J = np.meshgrid(np.arange(iv["m"]), np.arange(iv["n"]), indexing="ij")
        e = o.gemm_entries(iv["m"], iv["n"], iv["k"], float(g["alpha"][0]),
                           _nums(g["A"], dtype), iv["lda"], _nums(g["B"], dtype),
                           iv["ldb"], float(g["beta"][0]), _nums(g["C0"], dtype),
                           iv["ldc"], I.ravel(), J.ravel(), dtype=dtype)
        assert np.array_equal(e, want.ravel()), (dtype, e, want)
    g = read_golden("handworked_rowmajor.txt")
    iv = {k: int(g[k][0]) for k in ("N1", "N2", "N3", "lda", "ldb", "ldc")}
    R = o.matmat_rowmajor_f64(iv["lda"], iv["ldb"], iv["ldc"], _nums(g["A"], np.float64),
                              _nums(g["B"], np.float64), _nums(g["C0"], np.float64),
                              iv["N1"], iv["N2"], iv["N3"])
    want = _nums(g["R"], np.float64).reshape(iv["N1"], iv["N3"])
    assert np.array_equal(R, want), (R, want)
    I, J = np.meshgrid(np.arange(iv["N1"]), np.arange(iv["N3"]), indexing="ij")
    e = o.matmat_rowmajor_f64_entries(iv["lda"], iv["ldb"], iv["ldc"],
                                      _nums(g["A"], np.float64), _nums(g["B"], np.float64),
                                      _nums(g["C0"], np.float64), iv["N1"], iv["N2"],
                                      iv["N3"], I.ravel(), J.ravel())
    assert np.array_equal(e, want.ravel()), (e, want)


# --------------------------------------------------------- exact rationals
def _exact_check(R, exact, scale, kk):
    """|R - exact| <= gamma_{k+2} * scale, all in exact rational arithmetic."""
    g = gamma(kk + 2)
    for idx in np.ndindex(R.shape):
        r = R[idx]
        assert np.isfinite(r), (idx, r)
        err = abs(Fraction(float(r)) - exact[idx])
        assert err <= g * scale[idx], (idx, float(r), float(exact[idx]), float(err))


def _rand_scalar(rng, dtype):
    v = dtype(rng.uniform(-2.0, 2.0))
    return float(v)


def pin_exact_colmajor(o, seed=11, dtype=np.float32, max_dim=8, ld_extra=(0, 3)):
    """Brute force over all m, n, k in 1..max_dim against exact rationals."""
    rng = np.random.default_rng(seed)
    shapes = [(m, n, k) for m in range(1, max_dim + 1) for n in range(1, max_dim + 1)
              for k in range(1, max_dim + 1)]
    for t, (m, n, k) in enumerate(shapes):
        pad = ld_extra[t % len(ld_extra)]
        lda, ldb, ldc = m + pad, k + pad, m + pad
        Av = gi.draw(rng, m * k, "u", dtype)
        Bv = gi.draw(rng, k * n, "u", dtype)
        Cv = gi.draw(rng, m * n, "u", dtype)
        alpha = (1.0, _rand_scalar(rng, dtype))[t % 2]
        beta = (0.0, _rand_scalar(rng, dtype), 1.0)[t % 3]
        A = gi.colmajor(Av, m, k, lda, np.nan)
        B = gi.colmajor(Bv, k, n, ldb, np.nan)
        C = gi.colmajor(Cv, m, n, ldc, np.nan)
        R = o.gemm(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, dtype=dtype)
        Af = [[Fraction(float(Av[i + p * m])) for p in range(k)] for i in range(m)]
        Bf = [[Fraction(float(Bv[p + j * k])) for j in range(n)] for p in range(k)]
        fa, fb = Fraction(alpha), Fraction(beta)
        exact = np.empty((m, n), dtype=object)
        scale = np.empty((m, n), dtype=object)
        for i in range(m):
            for j in range(n):
                s = sum(Af[i][p] * Bf[p][j] for p in range(k))
                sa = sum(abs(Af[i][p] * Bf[p][j]) for p in range(k))
                c = Fraction(float(Cv[i + j * m]))
                exact[i, j] = fa * s + fb * c
                scale[i, j] = abs(fa) * sa + abs(fb) * abs(c)
        _exact_check(R, exact, scale, k)


def pin_exact_rowmajor(o, seed=12, max_dim=6):
    """Brute force of the row-major lecture form against exact rationals."""
    rng = np.random.default_rng(seed)
    t = 0
    for N1 in range(1, max_dim + 1):
        for N2 in range(1, max_dim + 1):
            for N3 in range(1, max_dim + 1):
                pad = (0, 2)[t % 2]
                lda, ldb, ldc = N2 + pad, N3 + pad, N3 + pad
                Av = gi.draw(rng, N1 * N2, "u", np.float64)
                Bv = gi.draw(rng, N2 * N3, "u", np.float64)
                Cv = gi.draw(rng, N1 * N3, "u", np.float64)
                alpha = (1.0, _rand_scalar(rng, np.float64))[t % 2]
                beta = (1.0, _rand_scalar(rng, np.float64), 0.0)[t % 3]
                A = gi.rowmajor(Av, N1, N2, lda, np.nan)
                B = gi.rowmajor(Bv, N2, N3, ldb, np.nan)
                C = gi.rowmajor(Cv, N1, N3, ldc, np.nan)
                R = o.matmat_rowmajor_f64(lda, ldb, ldc, A, B, C, N1, N2, N3,
                                          alpha=alpha, beta=beta)
                fa, fb = Fraction(alpha), Fraction(beta)
                exact = np.empty((N1, N3), dtype=object)
                scale = np.empty((N1, N3), dtype=object)
                for i in range(N1):
                    for j in range(N3):
                        prods = [Fraction(float(Av[i * N2 + p])) * Fraction(float(Bv[p * N3 + j]))
                                 for p in range(N2)]
                        c = Fraction(float(Cv[i * N3 + j]))
                        exact[i, j] = fa * sum(prods) + fb * c
                        scale[i, j] = abs(fa) * sum(abs(x) for x in prods) + abs(fb) * abs(c)
                _exact_check(R, exact, scale, N2)
                t += 1


# ------------------------------------------------------------ closed forms
def pin_identity(o):
    rng = gi.rng_for(21)
    for dtype in (np.float32, np.float64):
        for (m, n, ld_pad) in ((1, 1, 0), (7, 5, 2), (33, 17, 5), (64, 64, 0)):
            lda = m + ld_pad
            eye = np.zeros((m, m), dtype=dtype)
            np.fill_diagonal(eye, 1)
            A = gi.colmajor(eye.T.ravel(), m, m, lda, np.nan)
            Bv = gi.draw(rng, m * n, "u", dtype)
            Cv = gi.draw(rng, m * n, "u", dtype)
            B = gi.colmajor(Bv, m, n, m + 1, np.nan)
            C = gi.colmajor(Cv, m, n, m + 3, np.nan)
            R = o.gemm(m, n, m, 1.0, A, lda, B, m + 1, 0.0, C, m + 3, dtype=dtype)
            assert np.array_equal(R, Bv.reshape(n, m).T.astype(np.float64))
            R = o.gemm(m, n, m, 0.5, A, lda, B, m + 1, 2.0, C, m + 3, dtype=dtype)
            want = 0.5 * Bv.reshape(n, m).T.astype(np.float64) + \
                2.0 * Cv.reshape(n, m).T.astype(np.float64)
            assert np.array_equal(R, want)


def pin_closed_forms(o):
    for dtype in (np.float32, np.float64):
        for (m, n, k) in ((5, 3, 1), (4, 6, 777), (3, 2, 1000), (2, 2, 4096)):
            ones_a = gi.colmajor(np.ones(m * k, dtype), m, k, m + 1, np.nan)
            ones_b = gi.colmajor(np.ones(k * n, dtype), k, n, k + 2, np.nan)
            R = o.gemm(m, n, k, 1.0, ones_a, m + 1, ones_b, k + 2, 0.0, None, m, dtype=dtype)
            assert np.all(R == k), (m, n, k, R)
            # A(i,p) = p + 1, B = 1 -> k(k+1)/2
            ap = np.repeat(np.arange(1, k + 1, dtype=dtype), m)  # column p holds p+1
            A = gi.colmajor(ap, m, k, m, np.nan)
            R = o.gemm(m, n, k, 1.0, A, m, ones_b, k + 2, 0.0, None, m, dtype=dtype)
            assert np.all(R == k * (k + 1) // 2), (m, n, k)
            # A(i,p) = B(p,j) = p + 1 -> k(k+1)(2k+1)/6
            bp = np.tile(np.arange(1, k + 1, dtype=dtype), n)  # column j holds 1..k
            B = gi.colmajor(bp, k, n, k, np.nan)
            R = o.gemm(m, n, k, 1.0, A, m, B, k, 0.0, None, m, dtype=dtype)
            assert np.all(R == k * (k + 1) * (2 * k + 1) // 6), (m, n, k)
            # rank-1: A(i,p) = a_i, B(p,j) = b_j -> k * a_i * b_j
            a = np.arange(1, m + 1, dtype=dtype) - 3
            b = np.arange(1, n + 1, dtype=dtype) * 2 - 5
            A = gi.colmajor(np.tile(a, k), m, k, m, np.nan)
            B = gi.colmajor(np.repeat(b, k), k, n, k, np.nan)
            R = o.gemm(m, n, k, 1.0, A, m, B, k, 0.0, None, m, dtype=dtype)
            assert np.array_equal(R, k * np.outer(a, b).astype(np.float64)), (m, n, k)


def pin_transpose(o):
    """(A B)^T == B^T A^T bitwise: same products, same order in p."""
    rng = gi.rng_for(31)
    for dtype in (np.float32, np.float64):
        for (m, n, k) in ((9, 4, 13), (16, 31, 7), (1, 5, 3)):
            Av = gi.draw(rng, m * k, "u", dtype).reshape(k, m).T   # (m,k)
            Bv = gi.draw(rng, k * n, "u", dtype).reshape(n, k).T   # (k,n)
            A = gi.colmajor(Av.T.ravel(), m, k, m + 2, np.nan)
            B = gi.colmajor(Bv.T.ravel(), k, n, k + 1, np.nan)
            R = o.gemm(m, n, k, 1.0, A, m + 2, B, k + 1, 0.0, None, m, dtype=dtype)
            At = gi.colmajor(Av.ravel(), k, m, k + 3, np.nan)      # A^T, (k,m) col-major
            Bt = gi.colmajor(Bv.ravel(), n, k, n, np.nan)          # B^T, (n,k) col-major
            Rt = o.gemm(n, m, k, 1.0, Bt, n, At, k + 3, 0.0, None, n, dtype=dtype)
            assert np.array_equal(R, Rt.T), (m, n, k)


def pin_swap(o):
    """Row-major entry == column-major entry with operands swapped, bitwise."""
    rng = gi.rng_for(41)
    for (N1, N2, N3, pad) in ((5, 7, 3, 2), (12, 1, 9, 0), (20, 33, 17, 8)):
        lda, ldb, ldc = N2 + pad, N3 + pad + 1, N3 + pad
        A = gi.rowmajor(gi.draw(rng, N1 * N2, "u", np.float64), N1, N2, lda, np.nan)
        B = gi.rowmajor(gi.draw(rng, N2 * N3, "u", np.float64), N2, N3, ldb, np.nan)
        C = gi.rowmajor(gi.draw(rng, N1 * N3, "u", np.float64), N1, N3, ldc, np.nan)
        for (alpha, beta) in ((1.0, 1.0), (0.75, -1.25), (2.0, 0.0)):
            R = o.matmat_rowmajor_f64(lda, ldb, ldc, A, B, C, N1, N2, N3,
                                      alpha=alpha, beta=beta)
            # row-major X (r x c, ld) is column-major X^T (c x r, ld)
            Rc = o.gemm(N3, N1, N2, alpha, B, ldb, A, lda, beta, C, ldc,
                        dtype=np.float64)
            assert np.array_equal(R, Rc.T), (N1, N2, N3, alpha, beta)


def pin_linearity(o):
    rng = gi.rng_for(51)
    for dtype in (np.float32, np.float64):
        m, n, k = 23, 19, 41
        A = gi.colmajor(gi.draw(rng, m * k, "u", dtype), m, k, m, np.nan)
        B = gi.colmajor(gi.draw(rng, k * n, "u", dtype), k, n, k, np.nan)
        Cv = gi.draw(rng, m * n, "u", dtype)
        C = gi.colmajor(Cv, m, n, m, np.nan)
        C2 = Cv.reshape(n, m).T.astype(np.float64)
        R1 = o.gemm(m, n, k, 1.0, A, m, B, k, 0.0, None, m, dtype=dtype)
        R = o.gemm(m, n, k, 2.0, A, m, B, k, 0.5, C, m, dtype=dtype)
        assert np.array_equal(R, 2.0 * R1 + 0.5 * C2)
        R = o.gemm(m, n, k, -4.0, A, m, B, k, 0.0, C, m, dtype=dtype)
        assert np.array_equal(R, -4.0 * R1)
        for (alpha, beta) in ((0.75, -1.25), (1.5, 0.5), (-0.3, 0.7)):
            R = o.gemm(m, n, k, alpha, A, m, B, k, beta, C, m, dtype=dtype)
            want = alpha * R1 + beta * C2
            assert np.all(np.abs(R - want) <= 4 * np.spacing(np.abs(want) + 1e-300) + 1e-300)


def pin_numpy_special(o):
    rng = gi.rng_for(61)
    for dtype in (np.float32, np.float64):
        # K = 1: outer product, exact in double for fp32 inputs
        m, n = 37, 29
        a = gi.draw(rng, m, "u", dtype)
        b = gi.draw(rng, n, "u", dtype)
        R = o.gemm(m, n, 1, 1.0, a, m, b, 1, 0.0, None, m, dtype=dtype)
        want = np.outer(a.astype(np.float64), b.astype(np.float64))
        if dtype == np.float32:
            assert np.array_equal(R, want)
        else:
            assert np.array_equal(R, np.outer(a, b))
        # M = N = 1: dot product
        k = 501
        a = gi.draw(rng, k, "u", dtype)
        b = gi.draw(rng, k, "u", dtype)
        R = o.gemm(1, 1, k, 1.0, a, 1, b, k, 0.0, None, 1, dtype=dtype)
        d = np.dot(a.astype(np.float64), b.astype(np.float64))
        assert abs(R[0, 0] - d) <= 1e-13 * np.sum(np.abs(a.astype(np.float64) * b))
        # N = 1: matrix-vector product
        m, k = 45, 70
        Av = gi.draw(rng, m * k, "u", dtype)
        x = gi.draw(rng, k, "u", dtype)
        R = o.gemm(m, 1, k, 1.0, gi.colmajor(Av, m, k, m + 4, np.nan), m + 4, x, k,
                   0.0, None, m, dtype=dtype)
        Am = Av.reshape(k, m).T.astype(np.float64)
        want = Am @ x.astype(np.float64)
        assert np.allclose(R[:, 0], want, rtol=0, atol=1e-13 * k)
        # general: numpy float64 matmul of the widened inputs
        m, n, k = 61, 47, 83
        Av = gi.draw(rng, m * k, "n", dtype)
        Bv = gi.draw(rng, k * n, "n", dtype)
        Cv = gi.draw(rng, m * n, "n", dtype)
        R = o.gemm(m, n, k, 0.75, gi.colmajor(Av, m, k, m + 16, np.nan), m + 16,
                   gi.colmajor(Bv, k, n, k + 16, np.nan), k + 16, -1.25,
                   gi.colmajor(Cv, m, n, m + 16, np.nan), m + 16, dtype=dtype)
        Am = Av.reshape(k, m).T.astype(np.float64)
        Bm = Bv.reshape(n, k).T.astype(np.float64)
        Cm = Cv.reshape(n, m).T.astype(np.float64)
        want = 0.75 * (Am @ Bm) - 1.25 * Cm
        rel = np.linalg.norm(R - want) / np.linalg.norm(want)
        assert rel <= 1e-13, rel


def pin_not_read(o):
    """beta == 0 never reads C; alpha == 0 or k == 0 never reads A, B."""
    rng = gi.rng_for(71)
    for dtype in (np.float32, np.float64):
        m, n, k = 11, 7, 5
        A = gi.colmajor(gi.draw(rng, m * k, "u", dtype), m, k, m, np.nan)
        B = gi.colmajor(gi.draw(rng, k * n, "u", dtype), k, n, k, np.nan)
        Cn = np.full(m * n, np.nan, dtype=dtype)
        R = o.gemm(m, n, k, 1.0, A, m, B, k, 0.0, Cn, m, dtype=dtype)
        assert np.all(np.isfinite(R))
        Cv = gi.draw(rng, m * n, "u", dtype)
        An = np.full(m * k, np.nan, dtype=dtype)
        Bn = np.full(k * n, np.nan, dtype=dtype)
        R = o.gemm(m, n, k, 0.0, An, m, Bn, k, -2.0, Cv, m, dtype=dtype)
        assert np.array_equal(R, -2.0 * Cv.reshape(n, m).T.astype(np.float64))
        R = o.gemm(m, n, 0, 1.0, An, m, Bn, 1, 0.5, Cv, m, dtype=dtype)
        assert np.array_equal(R, 0.5 * Cv.reshape(n, m).T.astype(np.float64))
        R = o.gemm(m, n, 0, 1.0, An, m, Bn, 1, 0.0, Cn, m, dtype=dtype)
        assert np.array_equal(R, np.zeros((m, n)))
        assert o.gemm(0, n, k, 1.0, A, 1, B, k, 1.0, Cv, 1, dtype=dtype).shape == (0, n)
        assert o.gemm(m, 0, k, 1.0, A, m, B, k, 1.0, Cv, m, dtype=dtype).shape == (m, 0)


def pin_entries_match(o):
    """The one-entry-at-a-time form equals the full form bitwise."""
    rng = gi.rng_for(81)
    for dtype in (np.float32, np.float64):
        m, n, k = 50, 30, 77
        A = gi.colmajor(gi.draw(rng, m * k, "n", dtype), m, k, m + 5, np.nan)
        B = gi.colmajor(gi.draw(rng, k * n, "n", dtype), k, n, k + 1, np.nan)
        C = gi.colmajor(gi.draw(rng, m * n, "n", dtype), m, n, m + 2, np.nan)
        R = o.gemm(m, n, k, 0.75, A, m + 5, B, k + 1, -1.25, C, m + 2, dtype=dtype)
        I = rng.integers(0, m, 200)
        J = rng.integers(0, n, 200)
        e = o.gemm_entries(m, n, k, 0.75, A, m + 5, B, k + 1, -1.25, C, m + 2, I, J,
                           dtype=dtype)
        assert np.array_equal(e, R[I, J])
    N1, N2, N3 = 13, 21, 8
    A = gi.rowmajor(gi.draw(rng, N1 * N2, "u", np.float64), N1, N2, N2 + 3, np.nan)
    B = gi.rowmajor(gi.draw(rng, N2 * N3, "u", np.float64), N2, N3, N3 + 1, np.nan)
    C = gi.rowmajor(gi.draw(rng, N1 * N3, "u", np.float64), N1, N3, N3 + 2, np.nan)
    R = o.matmat_rowmajor_f64(N2 + 3, N3 + 1, N3 + 2, A, B, C, N1, N2, N3)
    I = rng.integers(0, N1, 60)
    J = rng.integers(0, N3, 60)
    e = o.matmat_rowmajor_f64_entries(N2 + 3, N3 + 1, N3 + 2, A, B, C, N1, N2, N3, I, J)
    assert np.array_equal(e, R[I, J])


ALL_PINS = [pin_golden, pin_exact_colmajor, pin_exact_rowmajor, pin_identity,
            pin_closed_forms, pin_transpose, pin_swap, pin_linearity,
            pin_numpy_special, pin_not_read, pin_entries_match]


def exact_colmajor_f64(o):
    pin_exact_colmajor(o, seed=13, dtype=np.float64, max_dim=6)


ALL_PINS.insert(2, exact_colmajor_f64)


def run_all(o, report=None):
    """Run every pin; return the list of names that failed.

    ``report`` (if given) is called with each failing pin's name as soon as
    it fails, so that a later crash in a broken build cannot hide it.
    """
    failed = []
    for pin in ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
            if report is not None:
                report(pin.__name__)
    return failed


if __name__ == "__main__":  # used by the mutation test, one build per process
    import oracle

    lib = oracle.OracleLib(sys.argv[1])
    failed = run_all(lib, report=lambda name: print("PIN-FAILED " + name, flush=True))
    sys.exit(1 if failed else 0)
