"""A call recorded into a HIP graph and replayed: once a stream has run a call
of a given shape (the work split is cached and the stream's workspace exists),
the same call is captured on that stream; every replay, with the program's
own work and synchronisations between replays, must give the bytes of the
eager call.  SYMV/HEMV with beta = 0 (y is not read, so each replay starts
from NaN in y) and the in-place triangular product (x reset before each
replay)."""
import numpy as np
import pytest

from blas_symmetric_mat_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def scalars(prec):
    if prec == "w":
        return (1.25, 2.0 ** -60), (0.0, 0.0)
    if prec in ("c", "z"):
        return complex(0.75, 0.25), 0.0
    return 1.25, 0.0


@pytest.mark.parametrize("prec", ["s", "d", "c", "z", "w"])
@pytest.mark.parametrize("uplo", ["L", "U"])
def test_symv_replayed_from_a_graph(prec, uplo):
    import torch
    import blas_symmetric_mat_amd as X
    G.log(f"graph replay {prec}{uplo}")
    al, be = scalars(prec)
    p = W.make_problem(prec, uplo, 3000, 3003, alpha=al, beta=be, seed=31)
    A, x = G.to_device(p.A), G.to_device(p.x)
    y = G.to_device(p.y)
    f = getattr(X, G.ENTRY[prec])
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        f(uplo, p.n, al, A, p.lda, x, 1, be, y, 1, stream=s)
    s.synchronize()
    eager = G.digest(y.cpu().numpy())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        f(uplo, p.n, al, A, p.lda, x, 1, be, y, 1, stream=s)
    for _ in range(4):
        y.fill_(float("nan"))  # beta = 0: y is never read
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert G.digest(y.cpu().numpy()) == eager


@pytest.mark.parametrize("prec", ["s", "z", "w"])
@pytest.mark.parametrize("uplo,trans", [("L", "N"), ("U", "C")])
def test_trmv_replayed_from_a_graph(prec, uplo, trans):
    import torch
    import blas_symmetric_mat_amd as X
    G.log(f"graph replay trmv {prec}{uplo}{trans}")
    p = W.make_trmv_problem(prec, uplo, trans, "N", 2500, 2501, seed=32)
    A = G.to_device(p.A)
    x0 = G.to_device(p.x)
    x = x0.clone()
    f = getattr(X, G.TENTRY[prec])
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        f(uplo, trans, "N", p.n, A, p.lda, x, 1, stream=s)
    s.synchronize()
    eager = G.digest(x.cpu().numpy())
    x.copy_(x0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        f(uplo, trans, "N", p.n, A, p.lda, x, 1, stream=s)
    for _ in range(4):
        x.copy_(x0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert G.digest(x.cpu().numpy()) == eager
    assert not np.array_equal(x.cpu().numpy(), p.x)
