"""Heavy cancellation in every row (S = kron(B, [[1, 1], [1, 1]]) + c*E with
x made of (v, -v) pairs, so that |S*x| is 1e-4 .. 1e-19 of |S||x|): the
oracle against exact rational arithmetic (CPU), and the device path against
both the exact result and the oracle (GPU), all within the componentwise
bound 4*n*eps*(|alpha||S||x| + |beta||y|).  For double-double the hi products
cancel exactly and every result comes from the lo words, which is where a
multiply-add with a single TwoSum of the high words is weakest."""
import numpy as np
import pytest

import oracle
from blas_symmetric_mat_amd import workloads as W
from tests import helpers as H

PRECS = ["s", "d", "c", "z", "w"]


def problem(prec, uplo, n, pad, seed):
    al = (1.5, 2.0 ** -60) if prec == "w" else (complex(0.75, 0.25) if prec in "cz" else 1.5)
    be = (0.0, 0.0) if prec == "w" else 0.0
    return W.make_cancelling_problem(prec, uplo, n, n + pad, seed=seed, alpha=al, beta=be)


def exact_ok(p, y):
    err = H.exact_errors(p, y)
    tol = H.tolerance(p)
    assert np.all(err <= tol), f"worst ratio {np.max(err / np.maximum(tol, 1e-300)):.3g}"


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("uplo", ["L", "U"])
def test_oracle_exact_under_cancellation(prec, uplo):
    p = problem(prec, uplo, 64, 3, seed=50)
    exact_ok(p, oracle.symv_problem(p))


def test_cancellation_is_heavy():
    """The inputs really cancel: |S*x| below 1e-3 of |S||x| in every row."""
    for prec in PRECS:
        p = problem(prec, "L", 64, 0, seed=51)
        ex = H.exact_result(p)
        mag = H.abs_bound_terms(p) / abs(complex(p.alpha if prec != "w" else p.alpha[0]))
        if prec in ("c", "z"):
            v = np.array([abs(complex(float(a), float(b))) for a, b in ex])
        else:
            v = np.array([abs(float(e)) for e in ex])
        assert np.all(v <= 1e-3 * mag), prec


@pytest.mark.gpu
@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("uplo", ["L", "U"])
def test_device_exact_under_cancellation(prec, uplo):
    from tests import gpu_util as G
    G.log(f"cancellation exact {prec}{uplo} n=258")
    p = problem(prec, uplo, 258, 5, seed=52)
    exact_ok(p, G.DeviceProblem(p).run())


@pytest.mark.gpu
@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("uplo", ["L", "U"])
def test_device_oracle_under_cancellation(prec, uplo):
    """n = 4098: several row strips of every type's configuration with a
    ragged last one; ten runs give identical bytes."""
    from tests import gpu_util as G
    G.log(f"cancellation oracle {prec}{uplo} n=4098")
    p = problem(prec, uplo, 4098, 2, seed=53)
    d = G.DeviceProblem(p)
    outs = [d.run() for _ in range(10)]
    assert len({G.digest(o) for o in outs}) == 1
    G.assert_close(p, outs[0], oracle.symv_problem(p), label=p.name)


@pytest.mark.gpu
@pytest.mark.parametrize("uplo", ["L", "U"])
def test_device_every_dd_strip_config_under_cancellation(uplo):
    """Every double-double row-strip configuration under heavy cancellation
    (the built-in rules reach only some of them at the sizes above): n = 258
    against the exact result, n = 1500 (several strips, a ragged last one)
    against the oracle, both within the componentwise bound."""
    import blas_symmetric_mat_amd as X
    from tests import gpu_util as G
    strips = [i for i in range(X.num_configs("w")) if X.config_info("w", i)["column_runs"] >= 4]
    assert strips
    small = problem("w", uplo, 258, 3, seed=54)
    big = problem("w", uplo, 1500, 1, seed=55)
    ref = oracle.symv_problem(big)
    try:
        for idx in strips:
            G.log(f"cancellation dd strip config #{idx} {uplo}")
            X.select_config("w", uplo, 0, 1 << 30, idx)
            exact_ok(small, G.DeviceProblem(small).run())
            G.assert_close(big, G.DeviceProblem(big).run(), ref, label=f"#{idx}")
    finally:
        X.select_config("w", uplo, 0, 1 << 30, -1)
