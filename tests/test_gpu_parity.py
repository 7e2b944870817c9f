"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, element by element, within
|y - y_ref| <= 4*n*eps*(|alpha||S||x| + |beta||y|) (eps = 2^-24, 2^-53,
2^-104), bitwise where the inputs make every summation order exact, and
bitwise identical from run to run."""
import numpy as np
import pytest

import oracle
from blas_symmetric_mat_amd import workloads as W
from tests import gpu_util as G
from tests import helpers as H

pytestmark = pytest.mark.gpu

PRECS = ("s", "d", "c", "z", "w")


def scalars(prec):
    if prec in ("c", "z"):
        return complex(0.75, 0.25), complex(0.5, -1.0)
    if prec == "w":
        return (1.5, 2.0 ** -60), (-0.5, 2.0 ** -58)
    return 1.5, -0.5


def problem(prec, uplo, n, pad=0, seed=0, **kw):
    al, be = scalars(prec)
    kw.setdefault("alpha", al)
    kw.setdefault("beta", be)
    if prec in ("c", "z"):
        kw.setdefault("diag_imag_scale", 1e3)
    return W.make_problem(prec, uplo, n, n + pad, seed=seed, **kw)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    G.torch_dev()
    import blas_symmetric_mat_amd as X
    G.log(f"library {X.version()} at {X.LIB_PATH}")


# ------------------------------------------------------------ random inputs

@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("n,pad", [(1, 0), (2, 0), (3, 1), (17, 0), (64, 0), (65, 3),
                                   (129, 0), (700, 5), (1024, 0), (1500, 2), (2111, 0)])
def test_parity_random(prec, uplo, n, pad):
    G.log(f"parity {prec} {uplo} n={n} lda={n + pad}")
    p = problem(prec, uplo, n, pad, seed=1000 + n)
    ref = oracle.symv_problem(p)
    got = G.DeviceProblem(p).run()
    G.assert_close(p, got, ref, label=f"{prec}{uplo}{n}")


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("n,pad", [(64, 0), (1000, 24), (2111, 1)])
def test_parity_integer_bitwise(prec, uplo, n, pad):
    """Integer-valued inputs: every summation order is exact, so the GPU must
    equal the oracle bit for bit (up to the sign of zero)."""
    G.log(f"integer {prec} {uplo} n={n}")
    p = W.make_integer_problem(prec, uplo, n, n + pad, seed=n)
    if prec in ("c", "z"):
        p.alpha, p.beta = complex(1.5, -0.5), complex(-0.5, 2.0)
    ref = oracle.symv_problem(p)
    got = G.DeviceProblem(p).run()
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("prec", PRECS)
def test_every_config(prec):
    """Every compiled tile configuration, both triangles, a size with several
    panels and tiles and ragged edges."""
    import blas_symmetric_mat_amd as X
    n = 1500
    try:
        for idx in range(X.num_configs(prec)):
            for uplo in "LU":
                X.select_config(prec, uplo, 0, 1 << 30, idx)
                G.log(f"config {prec} #{idx} {X.config_info(prec, idx)} {uplo}")
                p = problem(prec, uplo, n, 1, seed=idx)
                ref = oracle.symv_problem(p)
                got = G.DeviceProblem(p).run()
                G.assert_close(p, got, ref, label=f"{prec}{uplo} cfg{idx}")
                pi = W.make_integer_problem(prec, uplo, 700, 701, seed=idx)
                np.testing.assert_array_equal(G.DeviceProblem(pi).run(),
                                              oracle.symv_problem(pi))
    finally:
        for uplo in "LU":
            X.select_config(prec, uplo, 0, 1 << 30, -1)


# ------------------------------------------------------------- edge cases

@pytest.mark.parametrize("prec", PRECS)
def test_beta_zero_nan_y(prec):
    zero = (0.0, 0.0) if prec == "w" else 0.0
    p = problem(prec, "U", 333, 2, seed=5, beta=zero)
    ref = oracle.symv_problem(p, np.zeros_like(p.y))
    y_nan = np.full_like(p.y, np.nan)
    got = G.DeviceProblem(p).run(y_nan)
    assert np.all(np.isfinite(got))
    G.assert_close(p, got, ref, label="beta0")


@pytest.mark.parametrize("prec", PRECS)
def test_alpha_zero(prec):
    """alpha = 0: y := beta*y, A and x never read (both NaN)."""
    zero = (0.0, 0.0) if prec == "w" else 0.0
    be = (-0.5, 0.0) if prec == "w" else scalars(prec)[1]
    p = problem(prec, "L", 300, 0, seed=6, alpha=zero, beta=be)
    p.A[:] = np.nan
    p.x[:] = np.nan
    got = G.DeviceProblem(p).run()
    ref = oracle.symv_problem(p)
    # one rounding per real operation on both sides: identical bits
    if prec == "w":
        np.testing.assert_array_equal(got[:, 0] + got[:, 1], ref[:, 0] + ref[:, 1])
    else:
        np.testing.assert_array_equal(got, ref)
    # alpha = 0, beta = 1: y untouched, even NaN
    one = (1.0, 0.0) if prec == "w" else 1.0
    q = problem(prec, "L", 300, 0, seed=6, alpha=zero, beta=one)
    q.y[7] = np.nan
    np.testing.assert_array_equal(G.DeviceProblem(q).run(), q.y)


@pytest.mark.parametrize("prec", ["c", "z"])
@pytest.mark.parametrize("uplo", ["L", "U"])
def test_hermitian_diagonal_nan_imag(prec, uplo):
    """The imaginary words of the diagonal are never used: NaN there gives the
    same bits as zeros there."""
    p = problem(prec, uplo, 777, 0, seed=7)
    p.A.imag[W.diag_index(777, 777)] = np.nan
    got = G.DeviceProblem(p).run()
    q = problem(prec, uplo, 777, 0, seed=7)
    q.A.imag[W.diag_index(777, 777)] = 0
    np.testing.assert_array_equal(got, G.DeviceProblem(q).run())
    G.assert_close(q, got, oracle.symv_problem(q), label="diag")


@pytest.mark.parametrize("prec", PRECS)
def test_unreferenced_triangle_nan(prec):
    """NaN in the other triangle and in the padding rows never shows."""
    for uplo in "LU":
        p = problem(prec, uplo, 1100, 7, seed=8)
        q = problem(prec, uplo, 1100, 7, seed=8, fill=0.0)
        a = G.DeviceProblem(p).run()
        assert np.all(np.isfinite(a))
        np.testing.assert_array_equal(a, G.DeviceProblem(q).run())


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("incx,incy", [(-1, 1), (2, -3), (-2, 2)])
def test_increments(prec, incx, incy):
    n = 555
    p = problem(prec, "L", n, 0, seed=9)
    xs = W.empty(prec, n * abs(incx))
    ys = W.empty(prec, n * abs(incy))
    xs[H.vec_index(n, incx)] = p.x
    ys[H.vec_index(n, incy)] = p.y
    q = W.Problem(**{**p.__dict__})
    q.x, q.y, q.incx, q.incy = xs, ys, incx, incy
    got = G.DeviceProblem(q).run()
    ref = oracle.symv_problem(q)
    G.assert_close(q, got, ref, label="inc")
    # the gaps between strided elements are left alone
    mask = np.ones(len(ys), dtype=bool)
    mask[H.vec_index(n, incy)] = False
    assert np.all(np.isnan(got[mask]))
    # same bits as the unit-stride call on the gathered vectors
    np.testing.assert_array_equal(got[H.vec_index(n, incy)], G.DeviceProblem(p).run())


def test_argument_errors():
    import blas_symmetric_mat_amd as X
    torch = G.torch_dev()
    A = torch.zeros(16, dtype=torch.float64, device="cuda")
    x = torch.zeros(4, dtype=torch.float64, device="cuda")
    y = torch.zeros(4, dtype=torch.float64, device="cuda")
    cases = [(("X", 4, 1.0, A, 4, x, 1, 0.0, y, 1), -1),
             (("L", -1, 1.0, A, 4, x, 1, 0.0, y, 1), -2),
             (("L", 4, 1.0, None, 4, x, 1, 0.0, y, 1), -4),
             (("L", 4, 1.0, A, 3, x, 1, 0.0, y, 1), -5),
             (("L", 4, 1.0, A, 4, None, 1, 0.0, y, 1), -6),
             (("L", 4, 1.0, A, 4, x, 0, 0.0, y, 1), -7),
             (("L", 4, 1.0, A, 4, x, 1, 0.0, None, 1), -9),
             (("L", 4, 1.0, A, 4, x, 1, 0.0, y, 0), -10)]
    for args, code in cases:
        with pytest.raises(X.XsymvError) as e:
            X.xsymv_d(*args)
        assert e.value.code == code
    X.xsymv_d("L", 0, 1.0, None, 1, None, 1, 0.0, None, 1)


# ------------------------------------------------------------- determinism

@pytest.mark.parametrize("prec", PRECS)
def test_bitwise_repeatable(prec):
    """Ten runs, same inputs: identical bytes (no order-dependent atomics)."""
    for uplo in "LU":
        p = problem(prec, uplo, 2111, 0, seed=10)
        dp = G.DeviceProblem(p)
        digests = {G.digest(dp.run()) for _ in range(10)}
        assert len(digests) == 1


# ------------------------------------------------- caller-installed workspace

@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("uplo", ["L", "U"])
def test_installed_workspace(prec, uplo):
    """A workspace installed with xsymv_set_workspace gives bit-identical
    results to the library-owned one; one that is too small is refused with
    2000 before any device work (y untouched); removing it restores the
    library-owned workspace."""
    import torch
    import blas_symmetric_mat_amd as X
    n = 1500
    G.log(f"installed workspace {prec} {uplo} n={n}")
    p = problem(prec, uplo, n, 3, seed=77)
    d = G.DeviceProblem(p)
    ref = d.run()
    stream = torch.cuda.Stream()
    need = X.workspace_bytes(prec, uplo, n)
    assert 0 < need < 1 << 40
    buf = torch.empty(need, dtype=torch.uint8, device="cuda")
    small = torch.empty(need // 2, dtype=torch.uint8, device="cuda")
    try:
        with torch.cuda.stream(stream):
            X.set_workspace(buf, stream=stream)
            got = d.run()
            y0 = G.to_device(p.y)
            X.set_workspace(small, stream=stream)
            with pytest.raises(X.XsymvError) as e:
                d.run_device(y0)
            assert e.value.code == 2000
            torch.cuda.synchronize()
            assert G.digest(y0.cpu().numpy()) == G.digest(p.y)
            X.set_workspace(None, stream=stream)
            again = d.run()
    finally:
        X.set_workspace(None, stream=stream)
    assert G.digest(got) == G.digest(ref)
    assert G.digest(again) == G.digest(ref)


def test_read_bandwidth_reference():
    """The stream-read reference the benchmark divides by: positive, below the
    8 TB/s specification, the best launch at least the median, on a buffer of
    4 GiB (16 times the last-level cache) whose size is not a multiple of any
    layout's tile."""
    import blas_symmetric_mat_amd as X
    G.log("read bandwidth reference")
    med, best = X.read_bandwidth((4 << 30) + 4096 * 3, reps=3)
    assert 500.0 < med <= best and med < 8000.0, (med, best)
