"""gemm_f32_noalloc: gemm_f32_ws on the library's own fixed scratch array.

Through the C ABI on the GPU: consecutive calls (the second and third on
smaller inputs, so the array holds the previous call's partial sums when the
next one starts) each give exactly the bits of gemm_f32_ws with a fresh
workspace of pgemm_workspace_f32 bytes, and on exact-integer inputs exactly
the oracle's values; A, B, C and their guard bands are otherwise untouched.
"""
import os
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import gemm_inputs as gi  # noqa: E402
import oracle  # noqa: E402
from gpu_util import DevMat, assert_bitwise, assert_f32_parity, logical  # noqa: E402

torch = pytest.importorskip("torch")
pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]
pg = pytest.importorskip("precision_gemm_02_amd")


def say(*a):
    print("[noalloc]", *a, flush=True)


# (m, n, k, (lda, ldb, ldc), alpha, beta), largest first: a stream-K plan
# that fills most of the array (128 x 128 tiles, 240 workgroups), a smaller
# one (64 x 64 tiles with two K groups), and a shape with no stream-K.
CALLS = [
    (2150, 2030, 1000, (2151, 1001, 2153), 1.5, 0.5),
    (1145, 1171, 3840, (1148, 3840, 1148), 0.75, -1.25),
    (300, 200, 100, (301, 101, 303), 1.0, 0.0),
]


def run(p, entry):
    dA, dB, dC = DevMat(p.A), DevMat(p.B), DevMat(p.C)
    if entry == "noalloc":
        pg.gemm_f32_noalloc(p.m, p.n, p.k, p.alpha, dA.ptr, p.lda, dB.ptr, p.ldb, p.beta,
                            dC.ptr, p.ldc)
    else:
        need = pg.workspace_f32(p.m, p.n, p.k)
        dW = DevMat(np.zeros(max(1, need // 4), np.float32))
        pg.gemm_f32_ws(p.m, p.n, p.k, p.alpha, dA.ptr, p.lda, dB.ptr, p.ldb, p.beta, dC.ptr,
                       p.ldc, dW.ptr, need)
        torch.cuda.synchronize()
        dW.assert_untouched_outside(max(1, need // 4), 1, max(1, need // 4))
    torch.cuda.synchronize()
    dC.assert_untouched_outside(p.m, p.n, p.ldc)
    dA.assert_untouched_outside(p.m, p.k, p.lda)
    dB.assert_untouched_outside(p.k, p.n, p.ldb)
    return logical(dC.storage(), p.m, p.n, p.ldc).copy()


@pytest.mark.parametrize("dist", ["i2", "u"])
def test_noalloc_matches_workspace_entry_on_consecutive_calls(dist):
    needs = [pg.workspace_f32(m, n, k) for (m, n, k, *_r) in CALLS]
    assert needs[0] > needs[1] > needs[2] == 0, needs
    assert needs[0] <= pg.PGEMM_SCRATCH_BYTES
    problems = [gi.make_colmajor_problem("noalloc", np.float32, m, n, k, *lds, alpha, beta,
                                         seed=1200 + t, dist=dist,
                                         c_dist=None if beta == 0 else dist)
                for t, (m, n, k, lds, alpha, beta) in enumerate(CALLS)]
    got = []
    for p in problems:     # back to back on the one array, largest first
        say(dist, (p.m, p.n, p.k), "ws", pg.workspace_f32(p.m, p.n, p.k))
        got.append(run(p, "noalloc"))
    for p, g in zip(problems, got):
        want = run(p, "ws")
        assert np.array_equal(g.view(np.uint32), want.view(np.uint32)), (p.m, p.n, p.k)
        R = oracle.gemm(p.m, p.n, p.k, p.alpha, p.A, p.lda, p.B, p.ldb, p.beta, p.C, p.ldc)
        if dist == "i2":
            assert_bitwise(g, R)
        else:
            assert_f32_parity(g, R, p.k)
    # once more in the opposite order: the small call right after the large
    # one still reads only its own partial sums
    for p, g in zip(reversed(problems), reversed(got)):
        again = run(p, "noalloc")
        assert np.array_equal(again.view(np.uint32), g.view(np.uint32))


def test_noalloc_quick_returns_and_argument_codes():
    L = pg.library()
    dC = DevMat(np.ones(64, np.float32))
    assert L.gemm_f32_noalloc(0, 8, 8, 1.0, None, 1, None, 8, 0.0, dC.ptr, 1, None) == 0
    assert L.gemm_f32_noalloc(8, 8, 8, 1.0, dC.ptr, 7, dC.ptr, 8, 0.0, dC.ptr, 8, None) == -6
    torch.cuda.synchronize()
    assert np.array_equal(dC.fetch().view(np.uint32), dC.host_before.view(np.uint32))
