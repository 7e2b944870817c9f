"""GPU parity of xGEMV (y := alpha*op(A)*x + beta*y) through the C ABI
against the CPU oracle on the same seeded inputs: within
4*k*eps*(|alpha||op(A)||x| + |beta||y|), bitwise for integer inputs, and
bitwise identical from run to run."""
import numpy as np
import pytest

import oracle
from blas_symmetric_mat_amd import workloads as W
from tests import gpu_util as G
from tests import helpers as H

pytestmark = pytest.mark.gpu

PRECS = ("s", "d", "c", "z", "w")
TRANS = ("N", "T", "C")


def scalars(prec):
    if prec in ("c", "z"):
        return complex(0.75, 0.25), complex(0.5, -1.0)
    if prec == "w":
        return (1.5, 2.0 ** -60), (-0.5, 2.0 ** -58)
    return 1.5, -0.5


def problem(prec, trans, m, n, pad=0, seed=0, **kw):
    al, be = scalars(prec)
    kw.setdefault("alpha", al)
    kw.setdefault("beta", be)
    return W.make_gemv_problem(prec, trans, m, n, m + pad, seed=seed, **kw)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.torch_dev()
    import blas_symmetric_mat_amd as X
    G.log(f"library {X.version()} at {X.LIB_PATH}")


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("trans", TRANS)
@pytest.mark.parametrize("m,n,pad", [(1, 1, 0), (3, 5, 1), (64, 64, 0), (65, 130, 3),
                                     (700, 301, 5), (1500, 2111, 2), (2111, 1500, 0),
                                     (5000, 64, 1), (64, 5000, 0)])
def test_gemv_parity_random(prec, trans, m, n, pad):
    G.log(f"gemv parity {prec} {trans} m={m} n={n} lda={m + pad}")
    p = problem(prec, trans, m, n, pad, seed=2000 + m + 3 * n)
    ref = oracle.gemv_problem(p)
    got = G.GemvDevice(p).run()
    G.assert_close_gemv(p, got, ref, label=f"{prec}{trans}{m}x{n}")


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("trans", TRANS)
def test_gemv_integer_bitwise(prec, trans):
    G.log(f"gemv integer {prec} {trans}")
    p = problem(prec, trans, 1000, 700, 24, seed=7, integer=(-3, 3), alpha=1.5, beta=-0.5)
    got = G.GemvDevice(p).run()
    exp = H.gemv_integer_expected(p)
    assert G.digest(got[H.vec_index(p.leny, p.incy)]) == G.digest(exp)


@pytest.mark.parametrize("prec", PRECS)
def test_gemv_every_config(prec):
    import blas_symmetric_mat_amd as X
    try:
        for idx in range(X.gemv_num_configs(prec)):
            X.gemv_select_config(prec, idx)
            for trans in ("N", "C"):
                G.log(f"gemv config {prec} #{idx} {trans}")
                p = problem(prec, trans, 1531, 1203, 5, seed=idx)
                G.assert_close_gemv(p, G.GemvDevice(p).run(), oracle.gemv_problem(p),
                                    label=f"{prec}#{idx}{trans}")
    finally:
        X.gemv_select_config(prec, -1)


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("trans", ["N", "T"])
def test_gemv_beta_zero_nan_y(prec, trans):
    p = problem(prec, trans, 900, 333, 1, seed=3, beta=(0.0, 0.0) if prec == "w" else 0.0)
    p.y[:] = np.nan
    got = G.GemvDevice(p).run()
    G.assert_close_gemv(p, got, oracle.gemv_problem(p), label=f"{prec}{trans} beta0")


@pytest.mark.parametrize("prec", PRECS)
def test_gemv_alpha_zero_bitwise(prec):
    p = problem(prec, "N", 500, 300, 0, seed=4, alpha=(0.0, 0.0) if prec == "w" else 0.0)
    p.A[:] = np.nan
    p.x[:] = np.nan
    assert G.digest(G.GemvDevice(p).run()) == G.digest(oracle.gemv_problem(p))


@pytest.mark.parametrize("prec", PRECS)
def test_gemv_padding_nan_never_used(prec):
    p = problem(prec, "C", 777, 500, 9, seed=5)  # padding rows hold NaN
    got = G.GemvDevice(p).run()
    assert np.all(np.isfinite(got))
    G.assert_close_gemv(p, got, oracle.gemv_problem(p), label=f"{prec} padding")


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("trans", ["N", "C"])
@pytest.mark.parametrize("incx,incy", [(-1, 1), (2, -3)])
def test_gemv_increments(prec, trans, incx, incy):
    p = problem(prec, trans, 611, 402, 2, seed=6)
    lx, ly = p.lenx, p.leny
    xs = W.empty(prec, 1 + (lx - 1) * abs(incx))
    ys = W.empty(prec, 1 + (ly - 1) * abs(incy))
    xs[H.vec_index(lx, incx)] = p.x
    ys[H.vec_index(ly, incy)] = p.y
    q = W.GemvProblem(**{**p.__dict__, "x": xs, "y": ys, "incx": incx, "incy": incy})
    got = G.GemvDevice(q).run()
    ref = oracle.gemv_problem(q)
    G.assert_close_gemv(q, got, ref, label=f"{prec}{trans} inc {incx},{incy}")


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("trans", TRANS)
def test_gemv_bitwise_repeatable(prec, trans):
    p = problem(prec, trans, 3001, 2003, 1, seed=8)
    d = G.GemvDevice(p)
    digests = {G.digest(d.run()) for _ in range(10)}
    assert len(digests) == 1
