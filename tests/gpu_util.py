"""Helpers for GPU tests: guard-banded device buffers and comparisons.

Every matrix goes to the GPU inside a larger buffer whose margins hold a
sentinel bit pattern.  After a call the margins, and the leading-dimension
padding of C, must come back bit-identical: the library must never write
outside the logical block of C, and padding values must never reach C (A and
B padding holds NaN, which would poison any result it touched).
"""
from __future__ import annotations

import numpy as np

SENT32 = np.uint32(0x7FA5A5A5)           # a NaN bit pattern
SENT64 = np.uint64(0x7FF5A5A5A5A5A5A5)


def _bits(a):
    return a.view(np.uint32 if a.dtype == np.float32 else np.uint64)


class DevMat:
    """Storage array on the GPU with ``margin`` sentinel elements each side.

    ``offset`` elements of extra shift move the data pointer off 16-byte
    alignment (offset=1 with fp32 gives a 4-byte aligned pointer).
    """

    def __init__(self, storage: np.ndarray, margin: int = 64, offset: int = 0):
        import torch
        self.dtype = storage.dtype
        self.n = storage.size
        self.margin = margin + offset
        sent = SENT32 if self.dtype == np.float32 else SENT64
        host = np.empty(self.n + 2 * self.margin, dtype=self.dtype)
        _bits(host)[:] = sent
        host[self.margin:self.margin + self.n] = storage
        self.host_before = host.copy()
        self.t = torch.from_numpy(host).cuda()
        self.ptr = self.t.data_ptr() + self.margin * self.dtype.itemsize

    def fetch(self) -> np.ndarray:
        """Whole buffer (margins included) back on the host."""
        import torch
        torch.cuda.synchronize()
        return self.t.cpu().numpy()

    def storage(self) -> np.ndarray:
        return self.fetch()[self.margin:self.margin + self.n]

    def assert_untouched_outside(self, rows: int, cols: int, ld: int):
        """Margins and ld padding are bit-identical to what was uploaded."""
        now = self.fetch()
        b0, b1 = _bits(self.host_before), _bits(now)
        m = self.margin
        assert np.array_equal(b0[:m], b1[:m]), "write before the buffer"
        assert np.array_equal(b0[m + self.n:], b1[m + self.n:]), "write after the buffer"
        if cols and ld > rows:
            p0 = b0[m:m + ld * cols].reshape(cols, ld)[:, rows:]
            p1 = b1[m:m + ld * cols].reshape(cols, ld)[:, rows:]
            assert np.array_equal(p0, p1), "write into leading-dimension padding"


def logical(storage, rows, cols, ld):
    if rows == 0 or cols == 0:
        return np.zeros((rows, cols), dtype=storage.dtype)
    return storage[: ld * cols].reshape(cols, ld)[:, :rows].T


def assert_f32_parity(Cgpu: np.ndarray, R: np.ndarray, k: int):
    """max|dC| <= 1e-6*K and ||dC||_F / ||R||_F <= 1e-5 (fp32 tolerance)."""
    D = Cgpu.astype(np.float64) - R
    assert np.all(np.isfinite(Cgpu)), "non-finite output"
    maxabs = float(np.max(np.abs(D))) if D.size else 0.0
    nr = float(np.linalg.norm(R))
    rel = float(np.linalg.norm(D)) / nr if nr > 0 else float(np.linalg.norm(D))
    assert maxabs <= 1e-6 * max(k, 1), "max|dC| = %g > %g" % (maxabs, 1e-6 * max(k, 1))
    assert rel <= 1e-5, "relative Frobenius error %g > 1e-5" % rel
    return maxabs, rel


def assert_f64_parity(Cgpu: np.ndarray, R: np.ndarray):
    """||dC||_F / ||R||_F <= 1e-12 (fp64 tolerance)."""
    D = Cgpu - R
    assert np.all(np.isfinite(Cgpu)), "non-finite output"
    nr = float(np.linalg.norm(R))
    rel = float(np.linalg.norm(D)) / nr if nr > 0 else float(np.linalg.norm(D))
    assert rel <= 1e-12, "relative Frobenius error %g > 1e-12" % rel
    return rel


def assert_bitwise(Cgpu: np.ndarray, R: np.ndarray):
    """Exact-integer inputs: every summation order is exact, so equality."""
    got = Cgpu.astype(np.float64)
    bad = np.argwhere(got != R)
    assert bad.size == 0, "%d mismatches, first at %s: got %r want %r" % (
        len(bad), tuple(bad[0]), got[tuple(bad[0])], R[tuple(bad[0])])


def sample_indices(m, n, count, seed=0):
    """Random (I, J) plus the four corners and the last row and column."""
    rng = np.random.default_rng(seed)
    I = list(rng.integers(0, m, count))
    J = list(rng.integers(0, n, count))
    for (i, j) in ((0, 0), (m - 1, 0), (0, n - 1), (m - 1, n - 1)):
        I.append(i)
        J.append(j)
    for j in range(0, n, max(1, n // 64)):
        I.append(m - 1)
        J.append(j)
    for i in range(0, m, max(1, m // 64)):
        I.append(i)
        J.append(n - 1)
    return np.array(I, dtype=np.int64), np.array(J, dtype=np.int64)


def freivalds(Cgpu, A, B, C0, alpha, beta, vectors=4, seed=0):
    """max over random x in {-1,1}^n of ||C x - (alpha A (B x) + beta C0 x)|| / ||.||.

    A check of the whole output in O(n^2) per vector (Freivalds 1977),
    computed in float64 with numpy; independent of the oracle.
    """
    rng = np.random.default_rng(seed)
    worst = 0.0
    A64, B64 = A.astype(np.float64), B.astype(np.float64)
    C64 = Cgpu.astype(np.float64)
    C064 = None if beta == 0 else C0.astype(np.float64)
    for _ in range(vectors):
        x = rng.choice([-1.0, 1.0], size=Cgpu.shape[1])
        want = alpha * (A64 @ (B64 @ x))
        if C064 is not None:
            want = want + beta * (C064 @ x)
        got = C64 @ x
        worst = max(worst, float(np.linalg.norm(got - want) / np.linalg.norm(want)))
    return worst
