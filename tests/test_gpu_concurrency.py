"""Calls from several host threads, each on its own stream, at once: every
result must equal the same call made alone (bit for bit -- each call's
summation order depends only on its arguments and configuration), and the
per-stream workspaces must not mix.  Also a single stream whose calls need
growing workspaces, interleaved with smaller ones."""
import threading

import numpy as np
import pytest

from blas_symmetric_mat_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _jobs(seed):
    """A thread's calls: (kind, problem)."""
    return [("symv", W.make_problem("s", "L", 3001, 3003, alpha=1.25, beta=-0.5, seed=seed)),
            ("symv", W.make_problem("d", "U", 2500, 2500, alpha=0.75, beta=0.0, seed=seed + 1)),
            ("gemv", W.make_gemv_problem("s", "T", 2000, 1500, 2003, alpha=1.5, beta=0.25,
                                         seed=seed + 2)),
            ("trmv", W.make_trmv_problem("s", "L", "N", "N", 2222, 2230, seed=seed + 3)),
            ("symv", W.make_problem("z", "L", 1200, 1200, alpha=complex(0.5, 1.0),
                                    beta=complex(1.0, -0.5), seed=seed + 4))]


def _device(kind, p):
    if kind == "symv":
        return G.DeviceProblem(p)
    if kind == "gemv":
        return G.GemvDevice(p)
    return G.TrmvDevice(p)


def _run_uploaded(kind, d):
    """One call on the current stream; returns the output as a host array
    (synchronises only the current stream)."""
    import torch
    import blas_symmetric_mat_amd as X
    p = d.p
    if kind == "symv":
        y = G.to_device(p.y)
        getattr(X, G.ENTRY[p.prec])(p.uplo, p.n, p.alpha, d.A, p.lda, d.x, p.incx, p.beta, y,
                                    p.incy)
        out = y
    elif kind == "gemv":
        y = G.to_device(p.y)
        getattr(X, G.GENTRY[p.prec])(p.trans, p.m, p.n, p.alpha, d.A, p.lda, d.x, p.incx,
                                     p.beta, y, p.incy)
        out = y
    else:
        x = G.to_device(p.x)
        getattr(X, G.TENTRY[p.prec])(p.uplo, p.trans, p.diag, p.n, d.A, p.lda, x, p.incx)
        out = x
    torch.cuda.current_stream().synchronize()
    return out.cpu().numpy()


def test_threads_on_their_own_streams():
    import torch
    nthreads, rounds = 4, 6
    jobs = [_jobs(100 * t) for t in range(nthreads)]
    devs = [[(k, _device(k, p)) for k, p in js] for js in jobs]
    G.log("concurrency: reference calls, one at a time")
    want = [[G.digest(_run_uploaded(k, d)) for k, d in ds] for ds in devs]
    errors = []

    def worker(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for r in range(rounds):
                    for j, (k, d) in enumerate(devs[t]):
                        if G.digest(_run_uploaded(k, d)) != want[t][j]:
                            errors.append((t, r, j))
        except Exception as e:  # reported below
            errors.append((t, repr(e)))

    G.log(f"concurrency: {nthreads} threads x {rounds} rounds")
    ths = [threading.Thread(target=worker, args=(t,)) for t in range(nthreads)]
    for th in ths:
        th.start()
    for th in ths:
        th.join(timeout=240)
    assert not any(th.is_alive() for th in ths), "a worker thread did not finish"
    assert not errors, errors[:5]


def test_one_stream_growing_and_shrinking_workspace():
    """Calls alternating between small and large orders on one stream: the
    workspace grows (the old buffer is released only after the queued work
    is done) and every result equals its reference."""
    sizes = [300, 9000, 500, 20000, 1000, 12000]
    probs = [W.make_problem("d", "L", n, n, alpha=1.0, beta=0.5, seed=n) for n in sizes]
    devs = [G.DeviceProblem(p) for p in probs]
    ref = [G.digest(d.run()) for d in devs]
    import blas_symmetric_mat_amd as X
    X.release()  # start from an empty workspace
    for _ in range(2):
        for d, r in zip(devs, ref):
            assert G.digest(d.run()) == r


def test_size_queries_beside_running_calls():
    """Workspace-size queries (which fill the per-device cache of resident
    workgroup counts) from one thread while products run on other threads'
    streams: the queries answer consistently and the products keep their
    bytes."""
    import torch
    import blas_symmetric_mat_amd as X
    X.release()
    jobs = [_jobs(7000 + 100 * t) for t in range(2)]
    devs = [[(k, _device(k, p)) for k, p in js] for js in jobs]
    want = [[G.digest(_run_uploaded(k, d)) for k, d in ds] for ds in devs]
    queries = [lambda: X.workspace_bytes("s", "L", 3001),
               lambda: X.workspace_bytes("w", "U", 777),
               lambda: X.gemv_workspace_bytes("d", "T", 2000, 1500),
               lambda: X.trmv_workspace_bytes("c", "U", "N", 1500),
               lambda: X.shard_workspace_bytes("z", "L", 4000, 64, 4, 1),
               lambda: X.config_workgroups("d", 0, "U")]
    first = [q() for q in queries]
    errors = []
    stop = threading.Event()

    def runner(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for r in range(4):
                    for j, (k, d) in enumerate(devs[t]):
                        if G.digest(_run_uploaded(k, d)) != want[t][j]:
                            errors.append(("product", t, r, j))
        except Exception as e:  # reported below
            errors.append((t, repr(e)))

    def asker():
        try:
            while not stop.is_set():
                got = [q() for q in queries]
                if got != first:
                    errors.append(("query", got, first))
                    return
        except Exception as e:  # reported below
            errors.append(("asker", repr(e)))

    G.log("concurrency: size queries beside 2 product threads")
    ths = [threading.Thread(target=runner, args=(t,)) for t in range(2)]
    ask = threading.Thread(target=asker)
    ask.start()
    for th in ths:
        th.start()
    for th in ths:
        th.join(timeout=240)
    stop.set()
    ask.join(timeout=60)
    assert not any(th.is_alive() for th in ths + [ask]), "a thread did not finish"
    assert not errors, errors[:5]
