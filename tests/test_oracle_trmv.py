"""Pins of the triangular product oracle (xTRMV: x := op(T)*x with T the
stored triangle, unit or non-unit diagonal, op = T, T^T or T^H), another of
the Level-2 BLAS that the CUDA-xSYMV report's §5 points to.  Checked against
exact rational arithmetic, integer-exact inputs through int64 products, what
must not be read, increments, and the general product oracle on the
zero-filled triangle.
"""
import numpy as np
import pytest

from blas_symmetric_mat_amd import workloads as W
from tests import helpers as H

PRECS = ("s", "d", "c", "z", "w")
TRANS = ("N", "T", "C")


def problem(prec, uplo, trans, diag, n, pad=0, seed=0, **kw):
    return W.make_trmv_problem(prec, uplo, trans, diag, n, n + pad, seed=seed, **kw)


def RUN(lib, p):
    return lib.trmv_problem(p)


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("trans", TRANS)
@pytest.mark.parametrize("diag", ["N", "U"])
@pytest.mark.parametrize("n,pad", [(1, 0), (7, 2), (16, 3)])
def test_trmv_exact_bruteforce(prec, uplo, trans, diag, n, pad, oracle_lib):
    """Every output within 4*n*eps*(|op(T)||x|)_i of the exact product."""
    p = problem(prec, uplo, trans, diag, n, pad, seed=60 + n)
    x = RUN(oracle_lib, p)
    errs = H.trmv_exact_errors(p, x)
    tol = H.trmv_tolerance(p)
    assert np.all(errs <= tol), (errs - tol).max()


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("trans", TRANS)
@pytest.mark.parametrize("diag", ["N", "U"])
def test_trmv_integer_bitwise(prec, uplo, trans, diag, oracle_lib):
    """Integer T and x: every product and partial sum is exact, so the result
    equals the int64 product op(T)*x bit for bit."""
    n = 48
    p = problem(prec, uplo, trans, diag, n, 5, seed=11, integer=(-4, 4))
    x = RUN(oracle_lib, p)
    want = H.trmv_integer_expected(p)
    assert np.array_equal(x.view(np.uint8), want.view(np.uint8))


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("trans", TRANS)
def test_trmv_unit_diagonal_not_read(prec, uplo, trans, oracle_lib):
    """diag = 'U': NaN on the stored diagonal changes nothing: the result is
    within the bound of the exact product, and (s, d, c, z, where a product by
    one is exact) equals the non-unit product with ones on the diagonal.  A
    double-double product by one renormalises its operand, so there the two
    may differ in the last bits."""
    p = problem(prec, uplo, trans, "U", 21, 2, seed=12)
    q = W.TrmvProblem(**{**p.__dict__, "A": p.A.copy()})
    q.A[W.diag_index(p.n, p.lda)] = np.nan
    got = RUN(oracle_lib, q)
    ones = W.TrmvProblem(**{**p.__dict__, "A": p.A.copy(), "diag": "N"})
    one = (1.0, 0.0) if prec == "w" else 1.0
    ones.A[W.diag_index(p.n, p.lda)] = one
    want = RUN(oracle_lib, ones)
    assert np.all(np.isfinite(got))
    assert np.all(H.trmv_exact_errors(q, got) <= H.trmv_tolerance(q))
    if prec != "w":
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("trans", TRANS)
def test_trmv_other_triangle_not_read(prec, uplo, trans, oracle_lib):
    """NaN in the other triangle and the padding: the result stays finite, and
    equals the result with zeros there."""
    p = problem(prec, uplo, trans, "N", 19, 3, seed=13, fill=np.nan)
    got = RUN(oracle_lib, p)
    z = W.TrmvProblem(**{**p.__dict__, "A": np.nan_to_num(p.A, nan=0.0)})
    want = RUN(oracle_lib, z)
    assert np.all(np.isfinite(got))
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


@pytest.mark.parametrize("prec", ["s", "d", "w"])
@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("diag", ["N", "U"])
def test_trmv_real_conjugate_is_transpose(prec, uplo, diag, oracle_lib):
    p = problem(prec, uplo, "T", diag, 15, 1, seed=14)
    q = W.TrmvProblem(**{**p.__dict__, "trans": "C"})
    assert np.array_equal(RUN(oracle_lib, p).view(np.uint8), RUN(oracle_lib, q).view(np.uint8))


@pytest.mark.parametrize("prec", ["c", "z"])
@pytest.mark.parametrize("uplo", ["L", "U"])
def test_trmv_conjugate_transpose(prec, uplo, oracle_lib):
    """T^H x = conj(T^T conj(x)) exactly (conjugation only flips signs)."""
    p = problem(prec, uplo, "C", "N", 15, 1, seed=15)
    q = W.TrmvProblem(**{**p.__dict__, "trans": "T", "x": np.conj(p.x)})
    tc = RUN(oracle_lib, p)
    tt = RUN(oracle_lib, q)
    assert np.array_equal(tc, np.conj(tt))


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("trans", TRANS)
@pytest.mark.parametrize("incx", [-1, 3, -2])
def test_trmv_increments(prec, trans, incx, oracle_lib):
    """A strided x (either sign) gives the contiguous result at the strided
    positions and leaves the gaps untouched."""
    p = problem(prec, "L", trans, "N", 17, 2, seed=16)
    base = RUN(oracle_lib, p)
    xs = W.empty(prec, 1 + (p.n - 1) * abs(incx))
    xs[...] = 7.0
    idx = H.vec_index(p.n, incx)
    xs[idx] = p.x
    q = W.TrmvProblem(**{**p.__dict__, "x": xs, "incx": incx})
    got = RUN(oracle_lib, q)
    assert np.array_equal(got[idx].view(np.uint8), base.view(np.uint8))
    gaps = np.ones(len(xs), dtype=bool)
    gaps[idx] = False
    assert np.all(got[gaps] == 7.0)


@pytest.mark.parametrize("prec", ["s", "d", "c", "z"])
@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("trans", TRANS)
def test_trmv_is_gemv_of_the_zero_filled_triangle(prec, uplo, trans, oracle_lib):
    """The general product oracle (alpha = 1, beta = 0) on the triangle with
    zeros elsewhere gives the same bits: the added zero products are exact."""
    n = 23
    p = problem(prec, uplo, trans, "N", n, 2, seed=17)
    got = RUN(oracle_lib, p)
    A = np.nan_to_num(p.A, nan=0.0)
    g = W.GemvProblem(prec, trans, n, n, p.lda, 1.0, 0.0, A, p.x.copy(),
                      np.full(n, np.nan, dtype=p.x.dtype))
    want = oracle_lib.gemv_problem(g)
    assert np.allclose(got, want, rtol=0, atol=0)


@pytest.mark.parametrize("prec", PRECS)
def test_trmv_n_zero_and_one(prec, oracle_lib):
    """n = 1 is one product (real types: IEEE's correctly rounded a*x); n = 0
    returns at once and leaves x alone."""
    p = problem(prec, "U", "N", "N", 1, 0, seed=18)
    x = RUN(oracle_lib, p)
    if prec in ("s", "d"):
        assert x[0] == p.A[0] * p.x[0]
    assert H.trmv_exact_errors(p, x)[0] <= H.trmv_tolerance(p)[0]
    x0 = p.x.copy()
    x0[...] = np.nan
    assert oracle_lib.trmv(prec, "L", "N", "N", 0, p.A, 1, x0, 1) == 0
    assert np.all(np.isnan(x0))


def test_trmv_bad_arguments(oracle_lib):
    p = problem("d", "L", "N", "N", 4, 0, seed=0)
    base = dict(uplo="L", trans="N", diag="N", n=4, A=p.A, lda=4, x=p.x.copy(), incx=1)
    cases = [(dict(uplo="X"), -1), (dict(trans="X"), -2), (dict(diag="X"), -3),
             (dict(n=-1), -4), (dict(A=None), -5), (dict(lda=3), -6), (dict(x=None), -7),
             (dict(incx=0), -8)]
    for over, code in cases:
        k = {**base, **over}
        assert oracle_lib.trmv("d", k["uplo"], k["trans"], k["diag"], k["n"], k["A"], k["lda"],
                               k["x"], k["incx"]) == code
