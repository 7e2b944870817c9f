"""The device-side input drawer, run on the CPU device: the layout and the
distributions it promises (stored triangle finite and within [-1, 1], NaN in
the other strict triangle and the padding rows, double-double lo words at most
2^-53 of their hi words, Hermitian diagonal garbage within its scale), the
host copy, and the same values for the same seed."""
import numpy as np
import pytest

from blas_symmetric_mat_amd import workloads as W


def matrix_words(p):
    """(lda x n) word matrices of a host problem: (value, lo or None)."""
    if p.prec == "w":
        return (p.A[:, 0].reshape(p.n, p.lda).T, p.A[:, 1].reshape(p.n, p.lda).T)
    return p.A.reshape(p.n, p.lda).T, None


@pytest.mark.parametrize("prec", W.PRECISIONS)
@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("n,lda", [(1, 1), (7, 9), (40, 40)])
def test_device_draw_layout(prec, uplo, n, lda):
    pytest.importorskip("torch")
    scale = 5.0 if prec in ("c", "z") else None
    p = W.draw_on_device(prec, uplo, n, lda, seed=3, diag_imag_scale=scale, device="cpu")
    h = W.problem_to_host(p)
    assert isinstance(h.A, np.ndarray) and h.A.shape[0] == lda * n
    assert h.x.shape[0] == n and h.y.shape[0] == n
    M, lo = matrix_words(h)
    i, j = np.indices(M.shape)
    stored = ((i >= j) if uplo == "L" else (i <= j)) & (i < n)
    assert np.all(np.isfinite(M[stored]))
    assert np.all(np.isnan(M[~stored].real))
    re = M.real if prec in ("c", "z") else M
    assert np.all(np.abs(re[stored]) <= 1.0)
    if prec in ("c", "z"):
        d = np.diag(M[:n, :n])
        assert np.all(np.abs(d.imag) <= scale)
        off = stored & (i != j)
        assert np.all(np.abs(M[off].imag) <= 1.0)
    if prec == "w":
        assert np.all(np.abs(lo[stored]) <= np.abs(M[stored]) * 2.0 ** -53)
        for v in (h.x, h.y):
            assert np.all(np.abs(v[:, 1]) <= np.abs(v[:, 0]) * 2.0 ** -53)
    q = W.problem_to_host(W.draw_on_device(prec, uplo, n, lda, seed=3,
                                           diag_imag_scale=scale, device="cpu"))
    np.testing.assert_array_equal(q.A, h.A)
    np.testing.assert_array_equal(q.y, h.y)


def test_device_draw_spans_column_blocks():
    """Orders whose triangle is drawn in several column blocks keep the
    triangle boundary exact across block edges."""
    pytest.importorskip("torch")
    n, lda = 1100, 70000  # 2^26 words per block / lda = 958 columns: two blocks
    p = W.problem_to_host(W.draw_on_device("s", "L", n, lda, seed=1, device="cpu"))
    M, _ = matrix_words(p)
    i, j = np.indices((n, n))
    top = M[:n, :n]
    assert np.all(np.isfinite(top[i >= j])) and np.all(np.isnan(top[i < j]))
    assert np.all(np.isnan(M[n:, :]))


@pytest.mark.parametrize("prec", W.PRECISIONS)
@pytest.mark.parametrize("trans", ["N", "T"])
def test_device_draw_general(prec, trans):
    """The general-matrix drawer: A is m x n with lda = m and every element
    drawn, x and y have op(A)'s lengths, double-double lo words at most 2^-53
    of their hi words, and the same seed gives the same values."""
    pytest.importorskip("torch")
    m, n = 9, 6
    p = W.problem_to_host(W.gemv_on_device(prec, trans, m, n, seed=4, device="cpu"))
    assert p.lda == m and p.A.shape[0] == m * n
    assert (p.x.shape[0], p.y.shape[0]) == ((n, m) if trans == "N" else (m, n))
    for v in (p.A, p.x, p.y):
        hi = v[:, 0] if prec == "w" else v
        assert np.all(np.isfinite(hi)) and np.all(np.abs(hi.real) <= 1.0)
        if prec == "w":
            assert np.all(np.abs(v[:, 1]) <= np.abs(v[:, 0]) * 2.0 ** -53)
    q = W.problem_to_host(W.gemv_on_device(prec, trans, m, n, seed=4, device="cpu"))
    np.testing.assert_array_equal(q.A, p.A)
