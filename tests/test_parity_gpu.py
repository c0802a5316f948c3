"""GPU library vs the CPU oracle (needs an MI355X; every test is marked gpu).

Every call goes through the C ABI (``libpgemm.so`` via the thin binding).
Inputs come from ``gemm_inputs`` (seeded); expected values come only from
``oracle`` (or, for whole-output checks at the largest size, from Freivalds'
randomized identity computed with numpy).

Bars:
  * fp32: max|dC| <= 1e-6*K and ||dC||_F/||R||_F <= 1e-5;
  * fp64: ||dC||_F/||R||_F <= 1e-12;
  * exact-integer inputs (entries in {-2..2}, alpha/beta multiples of 1/4):
    every partial sum is an integer below 2^24, so every summation order is
    exact and the GPU must equal the oracle bit for bit;
  * C's leading-dimension padding and the guard margins around every buffer
    must be bit-identical after the call; A/B padding is NaN.
"""
import os
import re
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import gemm_inputs as gi  # noqa: E402
import oracle  # noqa: E402
from gpu_util import (DevMat, assert_bitwise, assert_f32_parity, assert_f64_parity,  # noqa: E402
                      freivalds, logical)

torch = pytest.importorskip("torch")
pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]
pg = pytest.importorskip("precision_gemm_02_amd")


def say(*a):
    print("[parity]", *a, flush=True)


def run_colmajor(p, offset=0, variant=None):
    """Run problem p (column-major) on the GPU; return (C logical, DevMats)."""
    dA, dB, dC = DevMat(p.A, offset=offset), DevMat(p.B), DevMat(p.C)
    if p.dtype == np.float32:
        fn = pg.gemm_f32 if variant is None else (
            lambda *a: pg.gemm_f32_variant(variant, *a))
    else:
        fn = pg.gemm_f64 if variant is None else (
            lambda *a: pg.gemm_f64_variant(variant, *a))
    fn(p.m, p.n, p.k, p.alpha, dA.ptr, p.lda, dB.ptr, p.ldb, p.beta, dC.ptr, p.ldc)
    torch.cuda.synchronize()
    dC.assert_untouched_outside(p.m, p.n, p.ldc)
    dA.assert_untouched_outside(p.m, p.k, p.lda)
    dB.assert_untouched_outside(p.k, p.n, p.ldb)
    return logical(dC.storage(), p.m, p.n, p.ldc).copy(), (dA, dB, dC)


def oracle_full(p):
    return oracle.gemm(p.m, p.n, p.k, p.alpha, p.A, p.lda, p.B, p.ldb, p.beta, p.C, p.ldc,
                       dtype=p.dtype)


# ------------------------------------------------------------- workloads
SMALL_WORKLOADS = ["sgemm_128", "sgemm_2048", "sgemm_sweep_512", "sgemm_sweep_1024",
                   "sgemm_sweep_2048", "sgemm_sweep_4096", "sgemm_ragged"]


@pytest.mark.parametrize("name", SMALL_WORKLOADS)
def test_workload_full_oracle(name):
    p = gi.workload(name)
    say(name, p.m, p.n, p.k, "variant", pg.select_f32(p.m, p.n, p.k, p.alpha, 1 << 20, p.lda,
                                                       1 << 20, p.ldb, p.beta, 1 << 20, p.ldc))
    C, _ = run_colmajor(p)
    R = oracle_full(p)
    maxabs, rel = assert_f32_parity(C, R, p.k)
    say(name, "max|dC| %.3g rel %.3g" % (maxabs, rel))


def test_workload_8192_full_oracle_and_freivalds():
    """The 8192^3 workload (alpha 1.5, beta 0.5): every one of the 8192^2
    entries against the full oracle (about 12 s on 16 host cores), plus
    Freivalds' check as an independent whole-output cross-check."""
    p = gi.workload("sgemm_sweep_8192")
    say("8192 generated")
    C, _ = run_colmajor(p)
    say("8192 gpu done; oracle ...")
    R = oracle_full(p)
    maxabs, rel = assert_f32_parity(C, R, p.k)
    say("8192 full oracle max|dC| %.3g rel %.3g" % (maxabs, rel))
    del R
    A = logical(p.A, p.m, p.k, p.lda)
    B = logical(p.B, p.k, p.n, p.ldb)
    C0 = logical(p.C, p.m, p.n, p.ldc)
    err = freivalds(C, A, B, C0, p.alpha, p.beta, vectors=3)
    say("8192 freivalds rel %.3g" % err)
    assert err <= 1e-5


def run_matmat(p):
    dA, dB, dC = DevMat(p.A), DevMat(p.B), DevMat(p.C)
    N1, N2, N3 = p.m, p.k, p.n
    pg.matmat_f64(p.lda, p.ldb, p.ldc, dA.ptr, dB.ptr, dC.ptr, N1, N2, N3)
    torch.cuda.synchronize()
    # row-major C (N1 x N3, ldc) is column-major (N3 x N1, ldc)
    dC.assert_untouched_outside(N3, N1, p.ldc)
    return gi.logical_rowmajor(dC.storage(), N1, N3, p.ldc).copy()


def test_workload_dgemm_rowmajor_full_oracle_and_freivalds():
    """The fp64 row-major 4096^3 workload (ld 4104, C += A*B) through
    matmat_f64: every entry against the row-major oracle (written from the
    lecture's formula, not through the operand swap), plus Freivalds' check."""
    p = gi.workload("dgemm_rowmajor")
    assert p.alpha == 1.0 and p.beta == 1.0   # the lecture's C += A*B
    C = run_matmat(p)
    N1, N2, N3 = p.m, p.k, p.n
    R = oracle.matmat_rowmajor_f64(p.lda, p.ldb, p.ldc, p.A, p.B, p.C, N1, N2, N3)
    rel = assert_f64_parity(C, R)
    say("dgemm 4096 full oracle rel %.3g" % rel)
    A = gi.logical_rowmajor(p.A, N1, N2, p.lda)
    B = gi.logical_rowmajor(p.B, N2, N3, p.ldb)
    C0 = gi.logical_rowmajor(p.C, N1, N3, p.ldc)
    err = freivalds(C, A, B, C0, 1.0, 1.0, vectors=3)
    say("dgemm 4096 freivalds rel %.3g" % err)
    assert err <= 1e-12


# the last two: N3 (the swapped problem's m) a few rows past whole 128-row
# tiles, so the strip kernel takes them (4 and 7 rows on 256 compute units)
@pytest.mark.parametrize("N1,N2,N3,pad", [(1, 1, 1, 0), (37, 53, 29, 8), (300, 257, 129, 2),
                                          (512, 512, 512, 8), (2244, 142, 1796, 0),
                                          (2047, 1501, 2055, 1)])
def test_matmat_f64_full_oracle(N1, N2, N3, pad):
    p = gi.make_rowmajor_problem("mm", N1, N2, N3, N2 + pad, N3 + pad, N3 + pad, 1.0, 1.0,
                                 seed=N1 + N2)
    C = run_matmat(p)
    R = oracle.matmat_rowmajor_f64(p.lda, p.ldb, p.ldc, p.A, p.B, p.C, N1, N2, N3)
    assert_f64_parity(C, R)


# --------------------------------------------------- exact-integer, bitwise
EXACT_SHAPES = [(1, 1, 1), (7, 5, 3), (32, 32, 8), (33, 65, 9), (256, 256, 64),
                (300, 260, 70), (513, 257, 1023), (129, 700, 31)]
ALPHA_BETA = [(1.0, 0.0), (1.0, 1.0), (0.75, -1.25), (1.5, 0.5)]


def exact_problem(dtype, m, n, k, alpha, beta, lds, seed):
    lda, ldb, ldc = lds
    return gi.make_colmajor_problem("exact", dtype, m, n, k, lda, ldb, ldc, alpha, beta,
                                    seed, dist="i2", c_dist=None if beta == 0 else "i2")


def variant_ids(prefix):
    return [v for v, n in pg.variants().items() if n.startswith(prefix)]


def leading_dims(m, k, vec, chunk, t):
    """Aligned ("vec") variants: multiples of the 16-byte chunk; unaligned: odd."""
    if vec:
        up = lambda x: -(-x // chunk) * chunk  # noqa: E731
        extra = chunk * (t % 2)
        return up(m) + extra, up(k) + extra, up(m) + 2 * extra
    return m + 1 + 2 * (t % 2), k + 1, m + 3


@pytest.mark.parametrize("variant", variant_ids("f32_") + variant_ids("f64_"),
                         ids=lambda v: pg.variants()[v])
def test_every_variant_exact_integer(variant):
    name = pg.variants()[variant]
    dtype = np.float32 if name.startswith("f32_") else np.float64
    chunk = 4 if dtype == np.float32 else 2
    vec = name.endswith("_vec")
    for t, (m, n, k) in enumerate(EXACT_SHAPES):
        alpha, beta = ALPHA_BETA[t % len(ALPHA_BETA)]
        lds = leading_dims(m, k, vec, chunk, t)
        p = exact_problem(dtype, m, n, k, alpha, beta, lds, seed=100 + t)
        say(name, (m, n, k), (alpha, beta), "ld", lds)
        C, _ = run_colmajor(p, variant=variant)
        assert_bitwise(C, oracle_full(p))


def ring_variants():
    out = []
    for v, n in pg.variants().items():
        m = re.match(r"f(32|64)_(\d+)x(\d+)x(\d+)_w\d+x\d+_s(\d+)(?:_k2)?_(vec|ua)$", n)
        if m and int(m.group(5)) > 2:
            out.append(v)
    return out


@pytest.mark.parametrize("variant", ring_variants(), ids=lambda v: pg.variants()[v])
def test_ring_pipeline_boundaries(variant):
    """K around the start and end of the branch-free steady-state loop
    (which runs while tile kt+S is whole), and tiles partly outside C."""
    name = pg.variants()[variant]
    m = re.match(r"f(32|64)_(\d+)x(\d+)x(\d+)_w\d+x\d+_s(\d+)(?:_k2)?_(vec|ua)$", name)
    prec, BM, BN, BK, S, kind = m.group(1), int(m.group(2)), int(m.group(3)), \
        int(m.group(4)), int(m.group(5)), m.group(6)
    dtype = np.float32 if prec == "32" else np.float64
    chunk = 4 if dtype == np.float32 else 2
    # whole K tiles nk: the steady-state loop runs nk - S iterations, first in
    # trips of S (compile-time stages), then 0..S-1 more with a runtime stage;
    # nk a multiple of S (2S, 3S) ends it at stage 0, where the last S tiles
    # take the compile-time drain
    Ks = sorted({1, BK - 1, BK * (S - 1), BK * S, BK * S + 1, BK * (S + 1) - 1,
                 BK * (S + 1), BK * (S + 1) + 1, BK * (S + 2) + 3, BK * 2 * S,
                 BK * (2 * S + 1), BK * (2 * S + 2), BK * (2 * S + 3), BK * 3 * S,
                 BK * (3 * S + 2) + 5})
    shapes = [(2 * BM, 2 * BN), (2 * BM + 5, BN + 3)]
    t = 0
    for (mm, nn) in shapes:
        for k in Ks:
            if k <= 0:
                continue
            lds = leading_dims(mm, k, kind == "vec", chunk, t)
            alpha, beta = ALPHA_BETA[t % len(ALPHA_BETA)]
            p = exact_problem(dtype, mm, nn, k, alpha, beta, lds, seed=200 + t)
            say(name, (mm, nn, k), (alpha, beta), "ld", lds)
            C, _ = run_colmajor(p, variant=variant)
            assert_bitwise(C, oracle_full(p))
            t += 1


@pytest.mark.parametrize("variant", [v for v in ring_variants()
                                     if pg.variants()[v].startswith("f64_")],
                         ids=lambda v: pg.variants()[v])
def test_f64_old_c_loaded_in_last_k_tiles(variant):
    """The fp64 kernels load a whole tile's old C during the last K tiles when
    beta != 0 and the tile lies inside C: in the compile-time drain when the
    steady state ends at stage 0 (K = 2*S*BK), in the loop over the last
    tiles otherwise (K = (2S+1)*BK, and with a K tail).  Every alpha/beta
    pair, whole and edge tiles; with beta = 0, C holds NaN and is never read."""
    name = pg.variants()[variant]
    m = re.match(r"f64_(\d+)x(\d+)x(\d+)_w\d+x\d+_s(\d+)_(vec|ua)$", name)
    BM, BN, BK, S, kind = (int(m.group(1)), int(m.group(2)), int(m.group(3)),
                           int(m.group(4)), m.group(5))
    t = 0
    for (mm, nn) in [(2 * BM, 2 * BN), (2 * BM + 3, BN + 5)]:
        for k in (BK * 2 * S, BK * (2 * S + 1), BK * (2 * S + 1) + 3):
            for alpha, beta in ALPHA_BETA:
                lds = leading_dims(mm, k, kind == "vec", 2, t)
                p = exact_problem(np.float64, mm, nn, k, alpha, beta, lds, seed=900 + t)
                if beta == 0:
                    p.C = gi.colmajor(np.full(mm * nn, np.nan), mm, nn, p.ldc,
                                      gi.C_SENTINEL_F64)
                say(name, (mm, nn, k), (alpha, beta), "ld", lds)
                C, _ = run_colmajor(p, variant=variant)
                assert_bitwise(C, oracle_full(p))
                if beta == 0:
                    assert not np.isnan(C).any()
                t += 1


@pytest.mark.parametrize("name", ["sgemm_128", "sgemm_2048", "sgemm_sweep_4096",
                                  "sgemm_ragged"])
def test_workload_shapes_exact_integer(name):
    p = gi.workload(name, dist_override="i2")
    if p.beta == 0:
        p.C = gi.colmajor(np.full(p.m * p.n, np.nan, np.float32), p.m, p.n, p.ldc,
                          gi.C_SENTINEL_F32)
    C, _ = run_colmajor(p)
    assert_bitwise(C, oracle_full(p))


def test_workload_8192_exact_integer_full():
    """8192^3 on exact-integer inputs with the workload's alpha and beta:
    every summation order is exact, so all 8192^2 entries equal the oracle."""
    p = gi.workload("sgemm_sweep_8192", dist_override="i2")
    C, _ = run_colmajor(p)
    assert_bitwise(C, oracle_full(p))


def test_dgemm_rowmajor_exact_integer_full():
    p = gi.workload("dgemm_rowmajor", dist_override="i2")
    C = run_matmat(p)
    assert_bitwise(C, oracle.matmat_rowmajor_f64(p.lda, p.ldb, p.ldc, p.A, p.B, p.C,
                                                 p.m, p.k, p.n))


# --------------------------------------------------------- special cases
@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_beta_zero_ignores_nan_c(dtype):
    p = gi.make_colmajor_problem("nanc", dtype, 200, 150, 77, 200, 80, 204, 1.0, 0.0, seed=3)
    assert np.isnan(logical(p.C, p.m, p.n, p.ldc)).all()
    C, _ = run_colmajor(p)
    R = oracle_full(p)
    if dtype == np.float32:
        assert_f32_parity(C, R, p.k)
    else:
        assert_f64_parity(C, R)


# Very long K loops on tiny outputs (thousands of K tiles, the K tail): the
# plain entry takes 32 x 32 tiles in four K groups, the workspace entry
# shares the K tiles by stream-K; integers in {-2..2} keep every partial sum
# exact (|sum| <= 4K < 2^24), so both must equal the oracle bitwise.
LONG_K_CASES = [
    (np.float32, 64, 64, 65537),
    (np.float32, 33, 7, 100003),
    (np.float32, 300, 200, 70001),
    (np.float64, 40, 50, 70001),
]


@pytest.mark.parametrize("case", range(len(LONG_K_CASES)))
def test_very_long_k_exact_integer(case):
    dtype, m, n, k = LONG_K_CASES[case]
    alpha, beta = ALPHA_BETA[case % len(ALPHA_BETA)]
    p = exact_problem(dtype, m, n, k, alpha, beta, (m + 1, k + 1, m + 2), seed=1700 + case)
    R = oracle_full(p)
    assert_bitwise(run_colmajor(p)[0], R)
    assert ws_size(p) > 0                  # stream-K: the K tiles are shared
    assert_bitwise(run_ws(p), R)
    say("long K", (m, n, k), (alpha, beta))


# Inf and NaN in A and B propagate as in IEEE arithmetic: with inputs from
# U[-1, 1) (no exact zeros, no overflow) every output is finite, +Inf, -Inf or
# NaN according to which non-finite values meet in its sum, whatever the
# summation order, so the kernels' classification must equal the oracle's
# element for element.  Shapes: 32 x 32 tiles in four K groups, 64 x 64 and
# 128 x 128 tiles with strip rows in the grid, 64 x 64 in two K groups with
# strip rows, 256 x 128 tiles, the stream-K path, fp64.
SPECIAL_CASES = [
    (np.float32, 200, 150, 77, False),
    (np.float32, 2051, 1000, 300, False),
    (np.float32, 4097, 3001, 1023, False),
    (np.float32, 391, 2418, 1564, False),
    (np.float32, 4097, 1500, 300, False),
    (np.float32, 2150, 2030, 1000, True),
    (np.float64, 700, 500, 99, False),
]


def _classify(C):
    out = np.zeros(C.shape, np.int8)
    out[np.isposinf(C)] = 1
    out[np.isneginf(C)] = 2
    out[np.isnan(C)] = 3
    return out


@pytest.mark.parametrize("case", range(len(SPECIAL_CASES)))
def test_inf_and_nan_propagate_like_the_oracle(case):
    dtype, m, n, k, use_ws = SPECIAL_CASES[case]
    p = gi.make_colmajor_problem("special", dtype, m, n, k, m + 1, k + 2, m + 3, 0.75, -1.25,
                                 seed=1500 + case, dist="u", c_dist="u")
    rng = np.random.default_rng(1600 + case)
    A = gi.logical_colmajor(p.A, m, k, p.lda).copy()
    B = gi.logical_colmajor(p.B, k, n, p.ldb).copy()
    for arr, count in ((A, 6), (B, 6)):
        for t in range(count):
            i, j = rng.integers(0, arr.shape[0]), rng.integers(0, arr.shape[1])
            arr[i, j] = (np.inf, -np.inf, np.nan)[t % 3]
    # the last row and column of A and B too (edge tiles, the K tail)
    A[m - 1, k - 1] = np.inf
    B[k - 1, n - 1] = -np.inf
    p.A = gi.colmajor(A.T.reshape(-1), m, k, p.lda, dtype(np.nan))
    p.B = gi.colmajor(B.T.reshape(-1), k, n, p.ldb, dtype(np.nan))
    R = oracle_full(p)
    C = run_ws(p) if use_ws else run_colmajor(p)[0]
    got, want = _classify(C), _classify(R)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (len(bad), bad[:4])
    fin = want == 0
    assert fin.sum() > m * n // 2          # most outputs stay finite
    if dtype == np.float32:
        assert_f32_parity(np.where(fin, C, 0), np.where(fin, R, 0), p.k)
    else:
        assert_f64_parity(np.where(fin, C, 0), np.where(fin, R, 0))
    say("special values", (m, n, k), "non-finite", int((~fin).sum()), "of", m * n)


# fp32: C = alpha*acc + beta*C is one fused multiply-add rounded once in fp32.
# With acc = 1 + 2^-23 (exact: only k = 0 contributes), alpha = 1,
# beta = 2^-24 (1 + 2^-23) and C = 1 - 2^-23, the exact result is
# 1 + 2^-23 + 2^-24 - 2^-70, just below the midpoint of 1 + 2^-23 and
# 1 + 2^-22: rounded once it is 1 + 2^-23; computed in double and rounded
# again it lands on the midpoint and ties to 1 + 2^-22.  One shape per path
# that computes the sum: small tiles, the 128 x 128 staged epilogue with the
# old C read during the last K tiles, strip rows in the grid's own
# workgroups, the strip kernel, and the stream-K fix-up.
ROUNDING_CASES = [
    ("small tiles", 64, 64, 16, (64, 16, 64), False, None),
    ("staged epilogue", 2048, 2048, 512, (2048, 512, 2048), False, "f32_128x128x16_w4x2_s4_vec"),
    ("strip in the grid", 4097, 3001, 1023, (4098, 1024, 4100), False, "strip"),
    ("strip kernel", 4357, 3791, 16, (4360, 16, 4360), False, "strip"),
    ("stream-K fix-up", 2150, 2030, 1000, (2150, 1000, 2150), True, "sk"),
]


@pytest.mark.parametrize("case", range(len(ROUNDING_CASES)), ids=lambda c: ROUNDING_CASES[c][0])
def test_fp32_epilogue_rounds_once(case):
    name, m, n, k, (lda, ldb, ldc), use_ws, path = ROUNDING_CASES[case]
    one_ulp = np.float32(1 + 2.0 ** -23)
    av = np.zeros((k, m), np.float32)
    av[0, :] = one_ulp                       # column 0 of A, column-major values
    bv = np.zeros((n, k), np.float32)
    bv[:, 0] = 1                             # row 0 of B
    cv = np.full(m * n, np.float32(1 - 2.0 ** -23))
    beta = float(np.float32(2.0 ** -24 * (1 + 2.0 ** -23)))
    p = gi.Problem("rounding", np.float32, m, n, k, lda, ldb, ldc, 1.0, beta,
                   gi.colmajor(av.reshape(-1), m, k, lda, np.float32(np.nan)),
                   gi.colmajor(bv.reshape(-1), k, n, ldb, np.float32(np.nan)),
                   gi.colmajor(cv, m, n, ldc, gi.C_SENTINEL_F32))
    if torch.cuda.get_device_properties(0).multi_processor_count == 256 and path is not None:
        dA, dB, dC = DevMat(p.A), DevMat(p.B), DevMat(p.C)
        v, sk, strip = pg.select_ws_f32(m, n, k, 1.0, dA.ptr, lda, dB.ptr, ldb, beta, dC.ptr,
                                        ldc, ws_size(p) if use_ws else 0)
        if path == "strip":
            assert strip > 0, (name, strip)
        elif path == "sk":
            assert sk > 0, (name, sk)
        else:
            assert pg.variants()[v] == path, pg.variants()[v]
    C = run_ws(p) if use_ws else run_colmajor(p)[0]
    want = np.float32(1 + 2.0 ** -23)
    bad = np.argwhere(C != want)
    assert bad.size == 0, (name, len(bad), bad[:4], C[tuple(bad[0])] if len(bad) else None)
    say("rounding", name, (m, n, k), "all", m * n, "elements", want)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_alpha_zero_and_k_zero_scale_c(dtype):
    m, n, ldc = 300, 70, 303
    rng = gi.rng_for(9)
    Cv = gi.draw(rng, m * n, "u", dtype)
    fn = pg.gemm_f32 if dtype == np.float32 else pg.gemm_f64
    for (k, alpha, beta) in ((0, 1.0, 0.5), (16, 0.0, -2.0), (0, 1.0, 0.0), (16, 0.0, 1.0)):
        dC = DevMat(gi.colmajor(Cv, m, n, ldc, gi.C_SENTINEL_F32 if dtype == np.float32
                                else gi.C_SENTINEL_F64))
        fn(m, n, k, alpha, None, m, None, max(k, 1), beta, dC.ptr, ldc)
        got = logical(dC.storage(), m, n, ldc)
        want = beta * logical(Cv.reshape(-1), m, n, m).astype(dtype) if beta != 0 else \
            np.zeros((m, n), dtype)
        assert np.array_equal(got, want.astype(dtype))
        dC.assert_untouched_outside(m, n, ldc)


def test_empty_shapes_touch_nothing():
    dC = DevMat(np.ones(64, np.float32))
    pg.gemm_f32(0, 8, 8, 1.0, None, 1, None, 8, 0.0, dC.ptr, 1)
    pg.gemm_f32(8, 0, 8, 1.0, None, 8, None, 8, 0.0, dC.ptr, 8)
    assert np.array_equal(dC.fetch().view(np.uint32), dC.host_before.view(np.uint32))


def test_unaligned_pointer_takes_unaligned_path():
    p = gi.make_colmajor_problem("unal", np.float32, 260, 130, 96, 260, 96, 260, 0.75, -1.25,
                                 seed=4, dist="n", c_dist="n")
    C, _ = run_colmajor(p, offset=1)  # A's pointer is only 4-byte aligned
    assert_f32_parity(C, oracle_full(p), p.k)


def test_device_info():
    """The device the library runs on, as the HIP runtime reports it: the
    compute-unit count agrees with torch's, and the peak clock is a plausible
    one (the MI355X's is 2.4 GHz)."""
    cus, khz = pg.device_info()
    assert cus == torch.cuda.get_device_properties(0).multi_processor_count
    assert 1_000_000 <= khz <= 4_000_000
    say("device", cus, "CUs at", khz / 1000, "MHz")


def test_determinism_bitwise():
    p = gi.workload("sgemm_2048")
    C1, _ = run_colmajor(p)
    C2, _ = run_colmajor(p)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))


def test_concurrent_calls_on_two_streams():
    """Two host threads, each with its own stream (and workspace), launch
    GEMMs concurrently: fp32 through gemm_f32_ws and fp64 through gemm_f64,
    eight times each on a fresh copy of C.  Every result is bitwise the one
    the same call gives alone: the library keeps no per-call state and its
    launches are ordered only by their own stream."""
    import threading
    p32 = exact_problem(np.float32, 2150, 2030, 1000, 1.5, 0.5, (2151, 1001, 2153), seed=700)
    p64 = exact_problem(np.float64, 900, 1100, 500, 0.75, -1.25, (901, 500, 902), seed=701)
    ref32 = oracle_full(p32)
    ref64 = oracle_full(p64)
    need = ws_size(p32)
    assert need > 0, "the fp32 case should take the stream-K path"
    jobs = []
    for p in (p32, p64):
        A = torch.from_numpy(p.A).cuda()
        B = torch.from_numpy(p.B).cuda()
        C0 = torch.from_numpy(p.C).cuda()
        jobs.append(dict(p=p, A=A, B=B, C0=C0, C=C0.clone(), s=torch.cuda.Stream()))
    W = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    errors = []

    def work(j):
        try:
            p, s = j["p"], j["s"]
            with torch.cuda.stream(s):
                for _ in range(8):
                    j["C"].copy_(j["C0"])
                    if p.dtype == np.float32:
                        pg.gemm_f32_ws(p.m, p.n, p.k, p.alpha, j["A"], p.lda, j["B"], p.ldb,
                                       p.beta, j["C"], p.ldc, W, need, stream=s)
                    else:
                        pg.gemm_f64(p.m, p.n, p.k, p.alpha, j["A"], p.lda, j["B"], p.ldb,
                                    p.beta, j["C"], p.ldc, stream=s)
            s.synchronize()
        except Exception as e:  # noqa: BLE001 (reported below)
            errors.append(e)

    threads = [threading.Thread(target=work, args=(j,)) for j in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for j, ref in zip(jobs, (ref32, ref64)):
        p = j["p"]
        got = logical(j["C"].cpu().numpy(), p.m, p.n, p.ldc)
        assert_bitwise(got, ref)


def test_linearity_bitwise():
    p = gi.make_colmajor_problem("lin", np.float32, 1000, 700, 300, 1000, 300, 1000, 1.0,
                                 0.0, seed=12, c_dist="u")
    C1, _ = run_colmajor(p)
    p.alpha, p.beta = 2.0, 0.5
    C2, _ = run_colmajor(p)
    C0 = logical(p.C, p.m, p.n, p.ldc)
    want = (np.float32(2.0) * C1 + np.float32(0.5) * C0).astype(np.float32)
    assert np.array_equal(C2.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_identity_and_closed_forms(dtype):
    m, n = 1000, 300
    eye = np.eye(m, dtype=dtype)
    Bv = gi.draw(gi.rng_for(13), m * n, "u", dtype)
    p = gi.Problem("eye", dtype, m, n, m, m, m, m, 1.0, 0.0,
                   eye.T.ravel().copy(), Bv.copy(), np.full(m * n, np.nan, dtype))
    C, _ = run_colmajor(p)
    assert np.array_equal(C, Bv.reshape(n, m).T)
    k = 5000
    p = gi.Problem("ones", dtype, 96, 80, k, 96, k, 96, 1.0, 0.0,
                   np.ones(96 * k, dtype), np.ones(k * 80, dtype), np.zeros(96 * 80, dtype))
    C, _ = run_colmajor(p)
    assert np.all(C == k)


def test_python_gemm_layouts():
    g = torch.Generator().manual_seed(0)
    A = torch.rand(333, 200, generator=g, dtype=torch.float32) * 2 - 1
    B = torch.rand(200, 150, generator=g, dtype=torch.float32) * 2 - 1
    C0 = torch.rand(333, 150, generator=g, dtype=torch.float32) * 2 - 1
    R = oracle.gemm(333, 150, 200, 0.5, A.t().contiguous().numpy().ravel(), 333,
                    B.t().contiguous().numpy().ravel(), 200, 2.0,
                    C0.t().contiguous().numpy().ravel(), 333)
    # row-major (contiguous) tensors: operand swap
    Cr = C0.clone().cuda()
    pg.gemm(A.cuda(), B.cuda(), Cr, alpha=0.5, beta=2.0)
    assert_f32_parity(Cr.cpu().numpy(), R, 200)
    # column-major views with padding
    Ap = torch.zeros(200, 340).cuda()   # storage of a 340-ld column-major A
    Ap[:, :333] = A.t().cuda()
    Acol = Ap.t()[:333, :]
    Ccol_store = torch.zeros(150, 336).cuda()
    Ccol_store[:, :333] = C0.t().cuda()
    Ccol = Ccol_store.t()[:333, :]
    Bcol = B.t().contiguous().cuda().t()
    pg.gemm(Acol, Bcol, Ccol, alpha=0.5, beta=2.0)
    assert_f32_parity(Ccol.cpu().numpy(), R, 200)
    assert torch.all(Ccol_store[:, 333:] == 0)
    # matrix-vector (n == 1), outer product (k == 1) and a row (m == 1), on
    # contiguous tensors: a dimension of size 1 fits either layout
    for (m, k, n) in ((333, 200, 1), (333, 1, 150), (1, 200, 150)):
        a, b, c0 = A[:m, :k].contiguous(), B[:k, :n].contiguous(), C0[:m, :n].contiguous()
        Rv = oracle.gemm(m, n, k, 0.5, a.t().contiguous().numpy().ravel(), m,
                         b.t().contiguous().numpy().ravel(), k, 2.0,
                         c0.t().contiguous().numpy().ravel(), m)
        cv = c0.cuda()
        pg.gemm(a.cuda(), b.cuda(), cv, alpha=0.5, beta=2.0)
        assert_f32_parity(cv.cpu().numpy(), Rv, k)
    # a CPU tensor is refused before anything is launched
    with pytest.raises(TypeError):
        pg.gemm(A, B.cuda(), C0.cuda())


# ------------------------- stream-K of the last round of tiles (workspace)
def ws_size(p):
    fn = pg.workspace_f32 if p.dtype == np.float32 else pg.workspace_f64
    return fn(p.m, p.n, p.k)


def run_ws(p, ws_bytes=None):
    """gemm_*_ws with a guard-banded workspace of ws_bytes (default: the size
    the library asks for); C, A, B and the workspace's margins are checked."""
    need = ws_size(p)
    nbytes = need if ws_bytes is None else ws_bytes
    item = np.dtype(p.dtype).itemsize
    welems = max(1, nbytes // item)
    dW = DevMat(np.zeros(welems, p.dtype))
    dA, dB, dC = DevMat(p.A), DevMat(p.B), DevMat(p.C)
    fn = pg.gemm_f32_ws if p.dtype == np.float32 else pg.gemm_f64_ws
    fn(p.m, p.n, p.k, p.alpha, dA.ptr, p.lda, dB.ptr, p.ldb, p.beta, dC.ptr, p.ldc,
       dW.ptr, nbytes)
    torch.cuda.synchronize()
    dC.assert_untouched_outside(p.m, p.n, p.ldc)
    dA.assert_untouched_outside(p.m, p.k, p.lda)
    dB.assert_untouched_outside(p.k, p.n, p.ldb)
    dW.assert_untouched_outside(welems, 1, welems)
    return logical(dC.storage(), p.m, p.n, p.ldc).copy()


# (dtype, m, n, k): each leaves a partly filled last round of tiles on 256
# compute units and so takes the stream-K path (tiling and plan as the
# library chooses them on 256 units: R full rounds + the rest, S stream-K
# workgroups; "aligned": no range crosses a tile; "crossing": some
# workgroups run two pieces).
# Together they cover every tile class with a stream-K form in both
# precisions, last rounds below and above half full and no full round at
# all, aligned and crossing plans, fewer workgroups than compute units,
# ragged M/N edges and K tails inside the shared tiles, and up to 50 pieces
# summed per tile.
SK_SHAPES = [
    (np.float32, 2150, 2030, 1000),    # 128^2: 256 + 16, S 240 aligned, K tail 8
    (np.float32, 3695, 1115, 669),     # 128^2: 256 + 5, S 50 aligned, K tail 13
    (np.float32, 2369, 2254, 1108),    # 128^2: 256 + 86, crossing, K tail 4
    (np.float32, 1351, 4463, 1130),    # 128^2: 256 + 129 (above half), crossing
    (np.float64, 1348, 3029, 2466),    # fp64 128^2: 256 + 8, 32 aligned pieces a tile
    (np.float64, 3196, 5224, 385),     # fp64 128^2: 4*256 + 1, S 6, K tail 1
    (np.float32, 2412, 539, 2591),     # 64^2: 256 + 86, crossing, K tail 15
    (np.float32, 231, 5532, 2524),     # 64^2: 256 + 92, crossing, K tail 12
    (np.float64, 200, 5553, 967),      # fp64 64^2: 256 + 92, crossing, K tail 7
    (np.float64, 9224, 73, 539),       # fp64 64^2: 256 + 34, S 238 aligned, K tail 11
    # no full round: every tile shared (at least 2 K tiles per workgroup)
    (np.float32, 67, 1116, 2269),      # 36 edge tiles of 64^2, crossing, K tail 13
    (np.float32, 66, 93, 1610),        # 4 edge tiles, S 200, 50 pieces each, K tail 10
    (np.float32, 1153, 76, 3027),      # 38 edge tiles, crossing, K tail 3
    (np.float64, 65, 2145, 1849),      # 68 fp64 edge tiles, crossing, K tail 9
    (np.float64, 136, 83, 606),        # 6 fp64 edge tiles, S 114, 19 pieces each
    # 64^2 with two K groups
    (np.float32, 1145, 1171, 3840),    # 256 + 86, crossing, unaligned ld
    (np.float32, 1399, 464, 5833),     # 176 tiles, no full round, crossing, K tail 9
    (np.float32, 5933, 138, 2931),     # 256 + 23, S 253, K tail 19
]


@pytest.mark.parametrize("case", range(len(SK_SHAPES)))
def test_stream_k_exact_integer(case):
    dtype, m, n, k = SK_SHAPES[case]
    alpha, beta = ALPHA_BETA[case % len(ALPHA_BETA)]
    chunk = 4 if dtype == np.float32 else 2
    lds = leading_dims(m, k, case % 2 == 0, chunk, case)
    p = exact_problem(dtype, m, n, k, alpha, beta, lds, seed=300 + case)
    assert ws_size(p) > 0, "shape no longer takes the stream-K path"
    say("stream-K", np.dtype(dtype).name, (m, n, k), (alpha, beta), "ld", lds, "ws", ws_size(p))
    C = run_ws(p)
    assert_bitwise(C, oracle_full(p))


def _random_cases(count, seed, mn_range=(1, 900), k_range=(1, 700)):
    """Seeded random problems: shapes, leading-dimension padding (odd or
    chunk-aligned), alpha/beta (zero included) and precision."""
    rng = np.random.default_rng(seed)
    cases = []
    for t in range(count):
        dtype = np.float32 if t % 3 else np.float64
        m, n = (int(x) for x in rng.integers(mn_range[0], mn_range[1], 2))
        k = int(rng.integers(k_range[0], k_range[1]))
        chunk = 4 if dtype == np.float32 else 2
        if rng.random() < 0.5:          # aligned: every ld a multiple of the chunk
            up = lambda x: -(-x // chunk) * chunk  # noqa: E731
            lds = (up(m) + chunk * int(rng.integers(0, 3)), up(k) + chunk * int(rng.integers(0, 3)),
                   up(m) + chunk * int(rng.integers(0, 3)))
        else:
            lds = (m + int(rng.integers(0, 5)), k + int(rng.integers(0, 5)), m + int(rng.integers(0, 5)))
        alpha, beta = ALPHA_BETA[int(rng.integers(0, len(ALPHA_BETA)))]
        if rng.random() < 0.1:
            alpha = 0.0
        cases.append((dtype, m, n, k, lds, alpha, beta))
    return cases


# small shapes (the 64 x 64 classes, most with stream-K over every tile) and
# mid-sized ones (every tile class, stream-K of a last round)
RANDOM_CASES = (_random_cases(48, seed=2024)
                + _random_cases(16, seed=2025, mn_range=(900, 2600), k_range=(1, 1200)))


@pytest.mark.parametrize("case", range(len(RANDOM_CASES)))
def test_random_shapes_every_entry_exact_integer(case):
    """The default entry point (whatever tile class its model picks) and the
    workspace entry point (with the stream-K plan it asks for) on seeded random small
    shapes, aligned or odd leading dimensions: bitwise equal to the oracle on
    exact-integer inputs, padding and guard bands untouched."""
    dtype, m, n, k, lds, alpha, beta = RANDOM_CASES[case]
    p = exact_problem(dtype, m, n, k, alpha, beta, lds, seed=600 + case)
    say("random", np.dtype(dtype).name, (m, n, k), (alpha, beta), "ld", lds, "ws", ws_size(p))
    R = oracle_full(p)
    C, _ = run_colmajor(p)
    assert_bitwise(C, R)
    if ws_size(p) > 0:
        assert_bitwise(run_ws(p), R)


# (dtype, m, n, k, (lda, ldb, ldc), the variant the default entry point picks
# on 256 compute units): one case per tile class and alignment, so that each
# class the shape choice can return runs through gemm_f32 / gemm_f64 itself.
CLASS_CASES = [
    (np.float32, 4096, 4096, 256, (4096, 256, 4096), "f32_256x256x16_w2x4_s3_vec"),
    (np.float32, 4097, 4095, 255, (4098, 256, 4100), "f32_256x256x16_w2x4_s3_ua"),
    (np.float32, 2047, 2047, 1023, (2048, 1024, 2050), "f32_128x128x16_w4x2_s4_ua"),
    (np.float32, 2560, 2560, 512, (2560, 512, 2560), "f32_256x128x32_w4x2_s3_vec"),
    (np.float32, 2561, 2559, 511, (2562, 512, 2564), "f32_256x128x32_w4x2_s3_ua"),
    (np.float32, 2048, 2048, 1024, (2052, 1028, 2056), "f32_128x128x16_w4x2_s4_vec"),
    (np.float32, 905, 893, 911, (906, 912, 908), "f32_64x64x16_w2x2_s4_ua"),
    (np.float32, 1000, 1000, 3000, (1000, 3000, 1000), "f32_64x64x32_w2x2_s3_k2_vec"),
    (np.float32, 1001, 999, 2500, (1002, 2501, 1004), "f32_64x64x32_w2x2_s3_k2_ua"),
    (np.float32, 512, 512, 512, (512, 512, 512), "f32_32x32x64_w1x1_s3_k4_vec"),
    (np.float32, 257, 301, 199, (258, 200, 259), "f32_32x32x64_w1x1_s3_k4_ua"),
    (np.float64, 2048, 2048, 512, (2050, 514, 2048), "f64_128x128x16_w2x4_s3_vec"),
    (np.float64, 2048, 2047, 511, (2049, 512, 2051), "f64_128x128x16_w2x4_s3_ua"),
    (np.float64, 700, 900, 500, (700, 500, 702), "f64_64x64x16_w2x4_s4_vec"),
    (np.float64, 701, 899, 501, (702, 501, 703), "f64_64x64x16_w2x4_s4_ua"),
]


@pytest.mark.parametrize("case", range(len(CLASS_CASES)), ids=lambda c: CLASS_CASES[c][5])
def test_every_tile_class_through_the_default_entry_exact_integer(case):
    dtype, m, n, k, lds, want = CLASS_CASES[case]
    alpha, beta = ALPHA_BETA[case % len(ALPHA_BETA)]
    p = exact_problem(dtype, m, n, k, alpha, beta, lds, seed=900 + case)
    dA, dB, dC = DevMat(p.A), DevMat(p.B), DevMat(p.C)
    sel = pg.select_f32 if dtype == np.float32 else pg.select_f64
    got = pg.variants()[sel(m, n, k, alpha, dA.ptr, p.lda, dB.ptr, p.ldb, beta, dC.ptr, p.ldc)]
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert got == want, (got, want)
    say("class", got, (m, n, k), lds, (alpha, beta))
    C, _ = run_colmajor(p)
    assert_bitwise(C, oracle_full(p))


# (dtype, m, n, k, (lda, ldb, ldc), workspace?, strip rows, stream-K?): a few
# rows below the last whole tile row go to the strip kernel (rows as the
# library chooses them on 256 compute units).  Every tile class under it,
# both alignments, K below the thread count (most threads without an inner
# index), column counts that leave the last workgroup 1 to 7 columns, and
# the workspace entry point (which asks for no workspace for these shapes).
STRIP_CASES = [
    (np.float32, 4097, 3001, 1023, (4098, 1024, 4100), False, 1, False),   # 128^2
    (np.float32, 2051, 2047, 1999, (2052, 2000, 2054), False, 3, False),   # K tail
    (np.float32, 4357, 3791, 16, (4360, 16, 4360), False, 5, False),       # 256^2, vec, K 16
    (np.float32, 3589, 2302, 36, (3590, 37, 3592), False, 5, False),       # 256x128, K 36
    (np.float32, 8199, 74, 655, (8200, 656, 8202), False, 7, False),       # 64^2
    (np.float32, 391, 2418, 1564, (392, 1565, 394), False, 7, False),      # 64^2, 2 K groups
    (np.float64, 2053, 4032, 157, (2054, 158, 2055), True, 5, False),      # workspace entry
    (np.float64, 1796, 2244, 142, (1796, 142, 1796), False, 4, False),     # fp64 128^2, vec
    (np.float64, 1926, 6455, 21, (1927, 22, 1928), False, 6, False),       # fp64 128^2, K 21
    (np.float64, 134, 5997, 230, (135, 231, 137), False, 6, False),        # fp64 64^2
    # strip rows and stream-K in one call (fp64 128^2 tiles: the fix-up
    # kernel sums the shared tiles of the first m - strip rows, the strip
    # kernel takes the rest)
    (np.float64, 1669, 5002, 3452, (1670, 3453, 1671), True, 5, True),     # odd ld
    (np.float64, 2181, 5884, 2761, (2182, 2762, 2184), True, 5, True),     # aligned (vec)
]


@pytest.mark.parametrize("case", range(len(STRIP_CASES)))
def test_strip_rows_exact_integer(case):
    dtype, m, n, k, lds, use_ws, rows, sk = STRIP_CASES[case]
    alpha, beta = ALPHA_BETA[case % len(ALPHA_BETA)]
    p = exact_problem(dtype, m, n, k, alpha, beta, lds, seed=950 + case)
    sel = pg.select_ws_f32 if dtype == np.float32 else pg.select_ws_f64
    dA, dB, dC = DevMat(p.A), DevMat(p.B), DevMat(p.C)
    v, sk_wgs, strip = sel(m, n, k, alpha, dA.ptr, p.lda, dB.ptr, p.ldb, beta, dC.ptr, p.ldc,
                           ws_size(p) if use_ws else 0)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert strip == rows and (sk_wgs > 0) == sk, (strip, sk_wgs)
    say("strip", pg.variants()[v], (m, n, k), lds, (alpha, beta), "rows", strip, "sk", sk_wgs)
    R = oracle_full(p)
    C = run_ws(p) if use_ws else run_colmajor(p)[0]
    assert_bitwise(C, R)


@pytest.mark.parametrize("case", [c for c in range(len(STRIP_CASES)) if STRIP_CASES[c][7]])
def test_strip_rows_with_stream_k_random_values(case):
    """The strip + stream-K cases on U[-1,1) values: within the fp64
    tolerance of the oracle, and run to run bitwise identical."""
    dtype, m, n, k, lds, use_ws, rows, sk = STRIP_CASES[case]
    p = gi.make_colmajor_problem("stripsk", dtype, m, n, k, *lds, 0.75, -1.25, seed=980 + case,
                                 dist="u", c_dist="u")
    C1 = run_ws(p)
    rel = assert_f64_parity(C1, oracle_full(p))
    C2 = run_ws(p)
    assert np.array_equal(C1.view(np.uint64), C2.view(np.uint64))
    say("strip+sk random", (m, n, k), "rel %.3g" % rel)


# (dtype, m, n, k, workspace?, strip rows, stream-K?): every path of the strip
# rows, as the library chooses them on 256 compute units -- each tile class
# under them (the 128 x 128 and 64 x 64 classes compute the strip in extra
# workgroups of their own grid, the others launch the strip kernel), every
# row count 1 to 8 that the class reaches, one column group per workgroup
# (each lane loads its own values of A) and several (the strip of A staged
# through LDS and shared), and with stream-K of the last round in the same
# call.
STRIP_PATH_CASES = [
    (np.float32, 2433, 3315, 118, False, 1, False),   # f32_128x128x16_w4x2_s4 r=1
    (np.float32, 385, 8563, 747, False, 1, False),   # f32_128x128x16_w4x2_s4 r=1, 4 column groups
    (np.float32, 769, 6909, 1324, True, 1, True),   # f32_128x128x16_w4x2_s4 r=1, 2 column groups, stream-K
    (np.float32, 4994, 1633, 73, False, 2, False),   # f32_128x128x16_w4x2_s4 r=2
    (np.float32, 1154, 6689, 112, False, 2, False),   # f32_128x128x16_w4x2_s4 r=2, 2 column groups
    (np.float32, 1794, 5268, 729, True, 2, True),   # f32_128x128x16_w4x2_s4 r=2, 2 column groups, stream-K
    (np.float32, 2691, 1494, 1820, False, 3, False),   # f32_128x128x16_w4x2_s4 r=3
    (np.float32, 1539, 5344, 14, False, 3, False),   # f32_128x128x16_w4x2_s4 r=3, 4 column groups
    (np.float32, 515, 8436, 1390, True, 3, True),   # f32_128x128x16_w4x2_s4 r=3, 4 column groups, stream-K
    (np.float32, 2436, 1607, 1492, False, 4, False),   # f32_128x128x16_w4x2_s4 r=4
    (np.float32, 772, 5340, 213, False, 4, False),   # f32_128x128x16_w4x2_s4 r=4, 4 column groups
    (np.float32, 772, 5511, 936, True, 4, True),   # f32_128x128x16_w4x2_s4 r=4, 4 column groups, stream-K
    (np.float32, 2693, 1448, 300, False, 5, False),   # f32_128x128x16_w4x2_s4 r=5
    (np.float32, 1541, 2645, 240, False, 5, False),   # f32_128x128x16_w4x2_s4 r=5, 2 column groups
    (np.float32, 1285, 3479, 1482, True, 5, True),   # f32_128x128x16_w4x2_s4 r=5, 4 column groups, stream-K
    (np.float32, 1926, 8657, 12, False, 6, False),   # f32_128x128x16_w4x2_s4 r=6, 8 column groups
    (np.float32, 1030, 4917, 739, True, 6, True),   # f32_128x128x16_w4x2_s4 r=6, 8 column groups, stream-K
    (np.float32, 1159, 3273, 476, False, 7, False),   # f32_128x128x16_w4x2_s4 r=7, 4 column groups
    (np.float32, 903, 4911, 1345, True, 7, True),   # f32_128x128x16_w4x2_s4 r=7, 8 column groups, stream-K
    (np.float32, 3464, 4721, 74, False, 8, False),   # f32_128x128x16_w4x2_s4 r=8, 8 column groups
    (np.float32, 1672, 5518, 903, True, 8, True),   # f32_128x128x16_w4x2_s4 r=8, 8 column groups, stream-K
    (np.float32, 3841, 4242, 10, False, 1, False),   # f32_256x256x16_w2x4_s3 r=1, 2 column groups
    (np.float32, 3843, 4231, 293, False, 3, False),   # f32_256x256x16_w2x4_s3 r=3, 2 column groups
    (np.float32, 1796, 8964, 305, False, 4, False),   # f32_256x256x16_w2x4_s3 r=4, 4 column groups
    (np.float32, 4872, 6431, 44, False, 8, False),   # f32_256x256x16_w2x4_s3 r=8, 4 column groups
    (np.float32, 577, 1610, 712, False, 1, False),   # f32_64x64x16_w2x2_s4 r=1
    (np.float32, 129, 8179, 482, False, 1, False),   # f32_64x64x16_w2x2_s4 r=1, 4 column groups
    (np.float32, 1026, 1021, 932, False, 2, False),   # f32_64x64x16_w2x2_s4 r=2
    (np.float32, 130, 6879, 399, False, 2, False),   # f32_64x64x16_w2x2_s4 r=2, 4 column groups
    (np.float32, 4675, 391, 947, False, 3, False),   # f32_64x64x16_w2x2_s4 r=3
    (np.float32, 195, 4738, 393, False, 3, False),   # f32_64x64x16_w2x2_s4 r=3, 4 column groups
    (np.float32, 3460, 840, 1464, False, 4, False),   # f32_64x64x16_w2x2_s4 r=4
    (np.float32, 260, 3942, 176, False, 4, False),   # f32_64x64x16_w2x2_s4 r=4, 4 column groups
    (np.float32, 453, 4499, 312, False, 5, False),   # f32_64x64x16_w2x2_s4 r=5, 4 column groups
    (np.float32, 454, 4243, 303, False, 6, False),   # f32_64x64x16_w2x2_s4 r=6, 4 column groups
    (np.float32, 2055, 508, 366, False, 7, False),   # f32_64x64x16_w2x2_s4 r=7
    (np.float32, 2183, 2340, 507, False, 7, False),   # f32_64x64x16_w2x2_s4 r=7, 4 column groups
    (np.float32, 4104, 202, 425, False, 8, False),   # f32_64x64x16_w2x2_s4 r=8
    (np.float32, 2504, 1608, 555, False, 8, False),   # f32_64x64x16_w2x2_s4 r=8, 4 column groups
    (np.float32, 1857, 1637, 2293, False, 1, False),   # f32_64x64x32_w2x2_s3_k2 r=1
    (np.float32, 129, 6010, 1547, False, 1, False),   # f32_64x64x32_w2x2_s3_k2 r=1, 4 column groups
    (np.float32, 2242, 1855, 1758, False, 2, False),   # f32_64x64x32_w2x2_s3_k2 r=2
    (np.float32, 194, 4259, 1610, False, 2, False),   # f32_64x64x32_w2x2_s3_k2 r=2
    (np.float32, 131, 5765, 539, False, 3, False),   # f32_64x64x32_w2x2_s3_k2 r=3, 8 column groups
    (np.float32, 1156, 895, 1809, False, 4, False),   # f32_64x64x32_w2x2_s3_k2 r=4
    (np.float32, 68, 8596, 751, False, 4, False),   # f32_64x64x32_w2x2_s3_k2 r=4, 8 column groups
    (np.float32, 197, 4236, 369, False, 5, False),   # f32_64x64x32_w2x2_s3_k2 r=5, 8 column groups
    (np.float32, 134, 6400, 600, False, 6, False),   # f32_64x64x32_w2x2_s3_k2 r=6
    (np.float32, 519, 3900, 800, False, 7, False),   # f32_64x64x32_w2x2_s3_k2 r=7
    (np.float32, 136, 5714, 271, False, 8, False),   # f32_64x64x32_w2x2_s3_k2 r=8, 8 column groups
    (np.float64, 2689, 1492, 631, False, 1, False),   # f64_128x128x16_w2x4_s3 r=1
    (np.float64, 4609, 6241, 34, False, 1, False),   # f64_128x128x16_w2x4_s3 r=1, 4 column groups
    (np.float64, 2562, 6501, 187, False, 2, False),   # f64_128x128x16_w2x4_s3 r=2, 4 column groups
    (np.float64, 1667, 7494, 39, False, 3, False),   # f64_128x128x16_w2x4_s3 r=3, 4 column groups
    (np.float64, 2308, 1747, 2049, False, 4, False),   # f64_128x128x16_w2x4_s3 r=4
    (np.float64, 4868, 8409, 12, False, 4, False),   # f64_128x128x16_w2x4_s3 r=4, 8 column groups
    (np.float64, 2949, 1402, 1971, False, 5, False),   # f64_128x128x16_w2x4_s3 r=5
    (np.float64, 3973, 4211, 132, False, 5, False),   # f64_128x128x16_w2x4_s3 r=5, 4 column groups
    (np.float64, 4614, 4453, 206, False, 6, False),   # f64_128x128x16_w2x4_s3 r=6, 8 column groups
    (np.float64, 4871, 5070, 53, False, 7, False),   # f64_128x128x16_w2x4_s3 r=7, 8 column groups
    (np.float64, 776, 5043, 469, False, 8, False),   # f64_128x128x16_w2x4_s3 r=8, 8 column groups
    (np.float64, 1217, 805, 1359, False, 1, False),   # f64_64x64x16_w2x4_s4 r=1
    (np.float64, 385, 2608, 885, False, 1, False),   # f64_64x64x16_w2x4_s4 r=1, 4 column groups
    (np.float64, 3458, 841, 546, False, 2, False),   # f64_64x64x16_w2x4_s4 r=2
    (np.float64, 642, 4858, 224, False, 2, False),   # f64_64x64x16_w2x4_s4 r=2, 8 column groups
    (np.float64, 194, 5684, 848, True, 2, True),   # f64_64x64x16_w2x4_s4 r=2, 8 column groups, stream-K
    (np.float64, 259, 3400, 120, False, 3, False),   # f64_64x64x16_w2x4_s4 r=3, 8 column groups
    (np.float64, 707, 3197, 802, True, 3, True),   # f64_64x64x16_w2x4_s4 r=3, 8 column groups, stream-K
    (np.float64, 132, 5777, 341, False, 4, False),   # f64_64x64x16_w2x4_s4 r=4, 8 column groups
    (np.float64, 133, 6554, 217, False, 5, False),   # f64_64x64x16_w2x4_s4 r=5, 8 column groups
    (np.float64, 134, 7771, 134, False, 6, False),   # f64_64x64x16_w2x4_s4 r=6, 8 column groups
    (np.float64, 390, 2883, 861, True, 6, True),   # f64_64x64x16_w2x4_s4 r=6, 8 column groups, stream-K
    (np.float64, 2311, 413, 1047, False, 7, False),   # f64_64x64x16_w2x4_s4 r=7
    (np.float64, 391, 4970, 175, False, 7, False),   # f64_64x64x16_w2x4_s4 r=7, 8 column groups
    (np.float64, 71, 2852, 1152, True, 7, True),   # f64_64x64x16_w2x4_s4 r=7, 8 column groups, stream-K
    (np.float64, 392, 2346, 616, False, 8, False),   # f64_64x64x16_w2x4_s4 r=8, 8 column groups
    (np.float64, 72, 2059, 1649, True, 8, True),   # f64_64x64x16_w2x4_s4 r=8, 8 column groups, stream-K
]


@pytest.mark.parametrize("case", range(len(STRIP_PATH_CASES)))
def test_strip_paths_exact_integer(case):
    dtype, m, n, k, use_ws, rows, sk = STRIP_PATH_CASES[case]
    alpha, beta = ALPHA_BETA[case % len(ALPHA_BETA)]
    chunk = 4 if dtype == np.float32 else 2
    lds = leading_dims(m, k, case % 2 == 1, chunk, case)
    p = exact_problem(dtype, m, n, k, alpha, beta, lds, seed=1300 + case)
    sel = pg.select_ws_f32 if dtype == np.float32 else pg.select_ws_f64
    dA, dB, dC = DevMat(p.A), DevMat(p.B), DevMat(p.C)
    v, sk_wgs, strip = sel(m, n, k, alpha, dA.ptr, p.lda, dB.ptr, p.ldb, beta, dC.ptr, p.ldc,
                           ws_size(p) if use_ws else 0)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert strip == rows and (sk_wgs > 0) == sk, (strip, sk_wgs)
    say("strip path", pg.variants()[v], (m, n, k), lds, (alpha, beta), "rows", strip, "sk",
        sk_wgs)
    C = run_ws(p) if use_ws else run_colmajor(p)[0]
    assert_bitwise(C, oracle_full(p))


def test_strip_rows_beta_zero_ignores_nan_in_c():
    """beta == 0: the strip rows, like the tiles, never read C."""
    p = exact_problem(np.float32, 4097, 3001, 1023, 1.0, 0.0, (4098, 1024, 4100), seed=970)
    R = oracle_full(p)            # C is zero here; with beta == 0 it does not matter
    p.C = np.full_like(p.C, np.nan)
    C, _ = run_colmajor(p)
    assert not np.isnan(C).any()
    assert_bitwise(C, R)


LONG_CASES = int(os.environ.get("PGEMM_LONG_TESTS", "0"))


@pytest.mark.skipif(LONG_CASES <= 0, reason="set PGEMM_LONG_TESTS=<count> to run")
def test_random_shapes_long():
    """Opt-in long run of the random-shape check (PGEMM_LONG_TESTS=3000 takes
    about two minutes): seeded problems up to 3000 x 3000 x 3000, both
    precisions, odd or aligned leading dimensions, alpha/beta including
    zero, through gemm_* and gemm_*_ws; bitwise against the oracle."""
    cases = (_random_cases(LONG_CASES * 7 // 10, seed=77)
             + _random_cases(LONG_CASES - LONG_CASES * 7 // 10, seed=78,
                             mn_range=(1, 3000), k_range=(1, 3000)))
    for t, (dtype, m, n, k, lds, alpha, beta) in enumerate(cases):
        p = exact_problem(dtype, m, n, k, alpha, beta, lds, seed=5000 + t)
        R = oracle_full(p)
        C, _ = run_colmajor(p)
        assert_bitwise(C, R)
        if ws_size(p) > 0:
            assert_bitwise(run_ws(p), R)
        if t % 250 == 0:
            say("long random", t, np.dtype(dtype).name, (m, n, k), lds, (alpha, beta))


def test_ragged_workload_strip_parity():
    """The ragged 4097 x 3001 x 1023 workload: 128 x 128 tiles on the first
    4096 rows (3 whole rounds) and the strip kernel on the last row, through
    both entry points (the workspace one asks for no workspace here)."""
    p = gi.workload("sgemm_ragged")
    dA, dB, dC = DevMat(p.A), DevMat(p.B), DevMat(p.C)
    v, sk, strip = pg.select_ws_f32(p.m, p.n, p.k, p.alpha, dA.ptr, p.lda, dB.ptr, p.ldb,
                                    p.beta, dC.ptr, p.ldc, ws_size(p))
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert strip == 1 and sk == 0 and ws_size(p) == 0
    C, _ = run_colmajor(p)
    maxabs, rel = assert_f32_parity(C, oracle_full(p), p.k)
    say("ragged", pg.variants()[v], "strip", strip, "max|dC| %.3g rel %.3g" % (maxabs, rel))
    assert np.array_equal(run_ws(p).view(np.uint32), C.view(np.uint32))
    q = gi.workload("sgemm_ragged", dist_override="i2")
    assert_bitwise(run_colmajor(q)[0], oracle_full(q))


def test_stream_k_fp64_parity():
    p = gi.make_colmajor_problem("sk64", np.float64, 200, 5553, 967, 201, 967, 203,
                                 0.75, -1.25, seed=31, dist="n", c_dist="n")
    assert ws_size(p) > 0
    assert_f64_parity(run_ws(p), oracle_full(p))


def test_stream_k_deterministic_and_small_workspace_is_plain():
    p = gi.make_colmajor_problem("skdet", np.float32, 2150, 2030, 1000, 2150, 1000, 2150,
                                 1.5, 0.5, seed=32, dist="u", c_dist="u")
    need = ws_size(p)
    C1, C2 = run_ws(p), run_ws(p)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))
    assert_f32_parity(C1, oracle_full(p), p.k)
    # a workspace one chunk short (or none) gives exactly gemm_f32's result
    plain, _ = run_colmajor(p)
    short = run_ws(p, ws_bytes=need - 16)
    assert np.array_equal(short.view(np.uint32), plain.view(np.uint32))
    none = run_ws(p, ws_bytes=0)
    assert np.array_equal(none.view(np.uint32), plain.view(np.uint32))


# ------------------------------------------------------ 64-bit addressing
def _big_storage(logical_cm, rows, cols, ld, dtype):
    """Device storage of a column-major (rows x cols) matrix with leading
    dimension ld (possibly > 2^31 elements in all), zeros elsewhere."""
    t = torch.zeros(ld * cols, dtype=dtype, device="cuda")
    t.view(cols, ld)[:, :rows] = torch.from_numpy(np.ascontiguousarray(logical_cm.T)).cuda()
    return t


@pytest.mark.parametrize("which,dtype", [("A", np.float32), ("B", np.float32), ("C", np.float32),
                                         ("C", np.float64)])
def test_storage_beyond_2_31_elements(which, dtype):
    """One operand's leading dimension puts its last columns more than 2^31
    elements (and 2^32 bytes) past its base: every address in the load and
    store paths must be formed in 64 bits."""
    tdt = torch.float32 if dtype == np.float32 else torch.float64
    m, n, k = 300, 2100, 2100
    big = 1 << 21                       # ld * 2100 columns > 2^32 elements
    lda, ldb, ldc = (big if which == "A" else m), (big if which == "B" else k), \
        (big if which == "C" else m)
    p = exact_problem(dtype, m, n, k, 0.75, -1.25, (m, k, m), seed=400)
    A = logical(p.A, m, k, m)
    B = logical(p.B, k, n, k)
    C0 = logical(p.C, m, n, m)
    say("64-bit", which, np.dtype(dtype).name, "ld", (lda, ldb, ldc))
    dA = _big_storage(A, m, k, lda, tdt)
    dB = _big_storage(B, k, n, ldb, tdt)
    dC = _big_storage(C0, m, n, ldc, tdt)
    fn = pg.gemm_f32 if dtype == np.float32 else pg.gemm_f64
    fn(m, n, k, p.alpha, dA, lda, dB, ldb, p.beta, dC, ldc)
    torch.cuda.synchronize()
    got = dC.view(n, ldc)[:, :m].t().cpu().numpy()
    pad = dC.view(n, ldc)[:, m:m + 64]
    assert bool((pad == 0).all()), "write into leading-dimension padding"
    del dA, dB, dC
    torch.cuda.empty_cache()
    assert_bitwise(got, oracle_full(p))


BUFFER_LIMIT_CASES = [
    # (variant, ldb): 256-column tiles reach BN*ldb + BK elements past the
    # tile's first column; 2^21 columns of fp32 cross 2^31 bytes (64-bit
    # masked loads), 2^21 - 64 stays just below (32-bit buffer offsets)
    ("f32_256x256x16_w2x4_s3_vec", 1 << 21), ("f32_256x256x16_w2x4_s3_vec", (1 << 21) - 64),
    ("f32_256x256x16_w2x4_s3_ua", (1 << 21) + 1), ("f32_256x256x16_w2x4_s3_ua", (1 << 21) - 63),
    ("f64_128x128x16_w2x4_s3_vec", 1 << 21), ("f64_128x128x16_w2x4_s3_vec", (1 << 21) - 32),
]


@pytest.mark.parametrize("name,ldb", BUFFER_LIMIT_CASES, ids=lambda x: str(x))
def test_whole_tile_loads_at_the_32_bit_offset_limit(name, ldb):
    """Whole-tile loads address each operand from its tile's first row or
    column with 32-bit byte offsets; when a leading dimension would take
    them past 2^31 bytes the kernel loads every tile with 64-bit masked
    addresses instead.  Both sides of the limit, edge tiles and a K tail."""
    dtype = np.float32 if name.startswith("f32_") else np.float64
    tdt = torch.float32 if dtype == np.float32 else torch.float64
    variant = [v for v, nm in pg.variants().items() if nm == name][0]
    m, n, k = 300, 260, 40
    lda, ldc = m + 1, m + 3
    if name.endswith("_vec"):
        lda, ldc = 304, 304
    p = exact_problem(dtype, m, n, k, 1.5, 0.5, (m, k, m), seed=450)
    A = logical(p.A, m, k, m)
    B = logical(p.B, k, n, k)
    C0 = logical(p.C, m, n, m)
    say("buffer limit", name, "ldb", ldb)
    dA = _big_storage(A, m, k, lda, tdt)
    dB = _big_storage(B, k, n, ldb, tdt)
    dC = _big_storage(C0, m, n, ldc, tdt)
    fn = pg.gemm_f32_variant if dtype == np.float32 else pg.gemm_f64_variant
    fn(variant, m, n, k, p.alpha, dA, lda, dB, ldb, p.beta, dC, ldc)
    torch.cuda.synchronize()
    got = dC.view(n, ldc)[:, :m].t().cpu().numpy()
    del dA, dB, dC
    torch.cuda.empty_cache()
    assert_bitwise(got, oracle_full(p))


# ------------------------------------------- lecture matmat on host memory
def run_matmat_host(p, pinned=False):
    """matmat_f64_host on host storage (copies of p's arrays); returns the
    logical C and the host buffers after the call."""
    N1, N2, N3 = p.m, p.k, p.n
    A, B, C = p.A.copy(), p.B.copy(), p.C.copy()
    if pinned:
        tA, tB, tC = (torch.from_numpy(x).pin_memory() for x in (A, B, C))
        A, B, C = tA.numpy(), tB.numpy(), tC.numpy()
    need = pg.matmat_host_workspace(p.lda, p.ldb, p.ldc, N1, N2, N3)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    pg.matmat_f64_host(p.lda, p.ldb, p.ldc, A, B, C, N1, N2, N3, ws, need)
    return gi.logical_rowmajor(C, N1, N3, p.ldc).copy(), (A, B, C)


@pytest.mark.parametrize("N1,N2,N3,pad", [(1, 1, 1, 0), (37, 53, 29, 8), (300, 257, 129, 3),
                                          (513, 300, 257, 0), (512, 512, 512, 8),
                                          (1000, 700, 1300, 1)])
def test_matmat_host_full_oracle(N1, N2, N3, pad):
    p = gi.make_rowmajor_problem("mmh", N1, N2, N3, N2 + pad, N3 + pad, N3 + pad, 1.0, 1.0,
                                 seed=N1 + 2 * N2)
    C, (A, B, Cbuf) = run_matmat_host(p)
    assert_f64_parity(C, oracle.matmat_rowmajor_f64(p.lda, p.ldb, p.ldc, p.A, p.B, p.C,
                                                    N1, N2, N3))
    # inputs untouched, C's row padding untouched (bit for bit)
    assert np.array_equal(A.view(np.uint64), p.A.view(np.uint64))
    assert np.array_equal(B.view(np.uint64), p.B.view(np.uint64))
    if pad:
        got_pad = Cbuf.reshape(N1, p.ldc)[:, N3:].view(np.uint64)
        want_pad = p.C.reshape(N1, p.ldc)[:, N3:].view(np.uint64)
        assert np.array_equal(got_pad, want_pad)


def test_matmat_host_equals_device_path():
    """Same kernel class on the same values: the host entry's result equals
    the device entry's bit for bit (exact-integer and random inputs, pinned
    and pageable host memory)."""
    for dist, pinned in (("i2", False), ("u", True)):
        p = gi.make_rowmajor_problem("mmh2", 777, 513, 901, 520, 905, 903, 1.0, 1.0, seed=41,
                                     dist=dist, c_dist=dist)
        Ch, _ = run_matmat_host(p, pinned=pinned)
        Cd = run_matmat(p)
        assert np.array_equal(Ch.view(np.uint64), Cd.view(np.uint64))
        if dist == "i2":
            assert_bitwise(Ch, oracle.matmat_rowmajor_f64(p.lda, p.ldb, p.ldc, p.A, p.B, p.C,
                                                          p.m, p.k, p.n))


# ------------------------------------------------ one GPU's share of 8192^3
def test_column_shard_of_8192_in_place():
    """The 8-GPU column split of the 8192^3 workload, shard 7, run in place on
    the full matrices: B and C by pointer offset (B + j0*ldb, C + j0*ldc),
    all of A.  Every entry of the shard matches the oracle (and Freivalds'
    check), and every column outside it is untouched."""
    full = gi.workload("sgemm_sweep_8192")
    p = gi.workload("sgemm_shard_8192_g8")
    j0 = gi.SHARD_COLUMN0[p.name]
    dA, dB, dC = DevMat(full.A), DevMat(full.B), DevMat(full.C)
    item = 4
    pg.gemm_f32(p.m, p.n, p.k, p.alpha, dA.ptr, p.lda, dB.ptr + j0 * p.ldb * item, p.ldb,
                p.beta, dC.ptr + j0 * p.ldc * item, p.ldc)
    torch.cuda.synchronize()
    store = dC.storage()
    before = full.C.view(np.uint32)
    assert np.array_equal(store[:j0 * p.ldc].view(np.uint32), before[:j0 * p.ldc]), \
        "columns before the shard changed"
    dC.assert_untouched_outside(full.m, full.n, full.ldc)
    C = logical(store[j0 * p.ldc:], p.m, p.n, p.ldc).copy()
    # the whole shard (8192 x 1024) through the full oracle, on the shard's
    # own pointers into the full-size B and C storage
    R = oracle.gemm(p.m, p.n, p.k, p.alpha, p.A, p.lda, p.B, p.ldb, p.beta, p.C, p.ldc)
    maxabs, rel = assert_f32_parity(C, R, p.k)
    say("shard full oracle max|dC| %.3g rel %.3g" % (maxabs, rel))
    err = freivalds(C, logical(p.A, p.m, p.k, p.lda), logical(p.B, p.k, p.n, p.ldb),
                    logical(p.C, p.m, p.n, p.ldc), p.alpha, p.beta, vectors=3)
    say("shard freivalds rel %.3g" % err)
    assert err <= 1e-5


# ---------------------------- edge tiles with tight leading dimensions
TIGHT_SHAPES = [(515, 257, 777), (3, 200, 900), (2, 100, 900), (1, 33, 600), (4095, 260, 300),
                (257, 130, 400)]


@pytest.mark.parametrize("variant", [v for v, n in pg.variants().items() if n.endswith("_ua")],
                         ids=lambda v: pg.variants()[v])
def test_tight_leading_dimension_edges_exact_integer(variant):
    """lda = m with m not a multiple of the 16-byte chunk: edge tiles read
    whole chunks across the end of a column (never in the last column), and
    tiny m takes the masked loads; C must match the oracle bit for bit."""
    name = pg.variants()[variant]
    dtype = np.float32 if name.startswith("f32_") else np.float64
    for t, (m, n, k) in enumerate(TIGHT_SHAPES):
        alpha, beta = ALPHA_BETA[t % len(ALPHA_BETA)]
        p = exact_problem(dtype, m, n, k, alpha, beta, (m, k, m), seed=500 + t)
        say(name, "tight", (m, n, k))
        C, _ = run_colmajor(p, variant=variant)
        assert_bitwise(C, oracle_full(p))
