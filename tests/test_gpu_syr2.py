"""GPU parity of the rank-2 update (xSYR2 / xHER2) through the C ABI against
the CPU oracle: for s, d, c, z the whole updated array (stored triangle,
untouched other triangle and padding) equals the oracle's byte for byte --
both take the BLAS reference order without fused multiply-adds; for
double-double (whose GPU product takes its cross terms with FMA) every stored
element is within 16*eps of its exact update and every other byte is
unchanged."""
import numpy as np
import pytest

import oracle
from blas_symmetric_mat_amd import workloads as W
from tests import gpu_util as G
from tests import test_oracle_syr2 as R2

pytestmark = pytest.mark.gpu

PRECS = ("s", "d", "c", "z", "w")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.torch_dev()


def check(p, label):
    got = G.run_syr2(p)
    ref = oracle.syr2_problem(p)
    if p.prec != "w":
        assert G.digest(got) == G.digest(ref), label
        return
    stored = np.zeros(p.A.shape[0], dtype=bool)
    for i, j in R2.stored_pairs(p):
        stored[i + j * p.lda] = True
    before = p.A.view(np.uint8).reshape(p.A.shape[0], -1)
    after = got.view(np.uint8).reshape(got.shape[0], -1)
    assert np.array_equal(before[~stored], after[~stored]), f"{label}: other triangle touched"
    if p.n <= 64:
        for (i, j), (v, scale) in R2.exact_update(p).items():
            err = R2.element_error("w", got[i + j * p.lda], v)
            assert err <= 16 * 2.0 ** -104 * scale, (label, i, j)
    else:
        # against the oracle: both within 16*eps of exact, so within 32*eps
        d = np.abs((got[stored, 0] - ref[stored, 0]) + (got[stored, 1] - ref[stored, 1]))
        scale = np.abs(p.A[stored, 0]) + 2 * 1.5 * 1.5  # |a| + |alpha|(|x||y| + |y||x|), |.| <= 1.5
        assert np.all(d <= 32 * 2.0 ** -104 * scale), label


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("n,pad", [(1, 0), (2, 1), (17, 0), (64, 3), (65, 0), (700, 5),
                                   (1500, 2), (2111, 0)])
def test_syr2_parity(prec, uplo, n, pad):
    G.log(f"syr2 {prec} {uplo} n={n} lda={n + pad}")
    p = R2.problem(prec, uplo, n, pad, seed=3000 + n, fill=123.5)
    check(p, f"{prec}{uplo}{n}")


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("uplo", ["L", "U"])
def test_syr2_nan_outside_triangle(prec, uplo):
    p = R2.problem(prec, uplo, 333, 7, seed=5)  # NaN in the other triangle and padding
    check(p, f"{prec}{uplo} NaN fill")


@pytest.mark.parametrize("prec", PRECS)
def test_syr2_every_config(prec):
    import blas_symmetric_mat_amd as X
    try:
        for idx in range(X.syr2_num_configs(prec)):
            X.syr2_select_config(prec, idx)
            for uplo in "LU":
                G.log(f"syr2 config {prec} #{idx} {uplo}")
                check(R2.problem(prec, uplo, 1203, 3, seed=idx, fill=-7.25),
                      f"{prec}#{idx}{uplo}")
    finally:
        X.syr2_select_config(prec, -1)


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("uplo", ["L", "U"])
def test_syr2_integer_bitwise(prec, uplo):
    p = W.make_syr2_problem(prec, uplo, 900, 903, alpha=1.5 if prec != "w" else (1.5, 0.0),
                            seed=9, integer=(-4, 4), fill=99.0)
    assert G.digest(G.run_syr2(p)) == G.digest(oracle.syr2_problem(p))


@pytest.mark.parametrize("prec", PRECS)
def test_syr2_alpha_zero_untouched(prec):
    p = R2.problem(prec, "U", 500, 2, seed=2, alpha=(0.0, 0.0) if prec == "w" else 0.0)
    p.x[:] = np.nan
    p.y[:] = np.nan
    assert G.digest(G.run_syr2(p)) == G.digest(p.A)


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("incx,incy", [(-1, 2), (3, -2)])
def test_syr2_increments(prec, incx, incy):
    p = R2.problem(prec, "L", 611, 1, seed=4, fill=5.5)
    xs = W.empty(prec, 1 + (p.n - 1) * abs(incx))
    ys = W.empty(prec, 1 + (p.n - 1) * abs(incy))
    from tests import helpers as H
    xs[H.vec_index(p.n, incx)] = p.x
    ys[H.vec_index(p.n, incy)] = p.y
    q = W.Syr2Problem(**{**p.__dict__, "x": xs, "y": ys, "incx": incx, "incy": incy})
    check(q, f"{prec} inc {incx},{incy}")
