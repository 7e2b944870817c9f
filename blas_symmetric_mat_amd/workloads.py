"""Seeded synthetic inputs for y := alpha*S*x + beta*y.

This module only draws numbers and lays them out; it holds none of the
product's arithmetic.  Both the GPU path's tests/benchmark and the CPU
oracle take their inputs from here, so the two always see the same data.

Layout (the BLAS layout of the CUDA-xSYMV report, §2.2 Fig. 5): A is a flat
column-major array of ``lda * n`` elements, element (i, j) at ``i + j*lda``.
Only the stored triangle (``uplo``) is drawn; the other strict triangle and
the padding rows ``n .. lda-1`` are filled with NaN, so that any read of them
would show in the result.

Element storage per precision code:
  's' float32, 'd' float64, 'c' complex64, 'z' complex128 (interleaved re, im),
  'w' double-double: float64 array with a trailing axis of 2 holding (hi, lo).

Drawing order for one problem, from ``numpy.random.Generator(PCG64(seed))``:
  1. the stored triangle, column by column (column-major), top to bottom;
  2. x (n values); 3. y (n values);
  4. Hermitian problems with diagonal garbage: n values that overwrite the
     imaginary words of the diagonal.
A complex value takes two consecutive draws (re, im).  A double-double value
takes two consecutive draws (r, r') and is hi = 2r-1, lo = hi*(2r'-1)*2^-53.
uniform[-1,1] is ``2*rng.random(dtype) - 1`` (exact in the element type);
normal is ``rng.standard_normal(dtype)``.
"""
from __future__ import annotations

import dataclasses
from typing import Any

import numpy as np

PRECISIONS = ("s", "d", "c", "z", "w")

# element dtype, real dtype, bytes per element
_DTYPE = {
    "s": (np.float32, np.float32, 4),
    "d": (np.float64, np.float64, 8),
    "c": (np.complex64, np.float32, 8),
    "z": (np.complex128, np.float64, 16),
    "w": (np.float64, np.float64, 16),
}


def elem_bytes(prec: str) -> int:
    return _DTYPE[prec][2]


def real_dtype(prec: str):
    return _DTYPE[prec][1]


def empty(prec: str, count: int, fill: float = np.nan) -> np.ndarray:
    """Array of ``count`` elements of type ``prec`` filled with ``fill``."""
    if prec == "w":
        return np.full((count, 2), fill, dtype=np.float64)
    if prec in ("c", "z"):
        return np.full(count, complex(fill, fill), dtype=_DTYPE[prec][0])
    return np.full(count, fill, dtype=_DTYPE[prec][0])


def _flat_real(a: np.ndarray) -> np.ndarray:
    """Contiguous real view of an element array (complex: (re, im) words;
    double-double: (hi, lo) words)."""
    if a.dtype in (np.complex64, np.complex128):
        return a.view(a.real.dtype)
    return a.reshape(-1)


def draw_into(rng: np.random.Generator, prec: str, out: np.ndarray,
              dist: str = "uniform", scale: float = 1.0) -> np.ndarray:
    """Fill the contiguous element array ``out`` with draws from ``dist``
    ('uniform' on [-scale, scale] or 'normal'), in place."""
    rdt = _DTYPE[prec][1]
    raw = _flat_real(out)
    if dist == "uniform":
        rng.random(out=raw, dtype=rdt)
        raw *= rdt(2)
        raw -= rdt(1)
    elif dist == "normal":
        rng.standard_normal(out=raw, dtype=rdt)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    if scale != 1.0:
        raw *= rdt(scale)
    if prec == "w":
        # pairs (hi, u) -> (hi, hi*u*2^-53)
        out[:, 1] *= out[:, 0]
        out[:, 1] *= 2.0 ** -53
    return out


def draw(rng: np.random.Generator, prec: str, count: int, dist: str = "uniform",
         scale: float = 1.0) -> np.ndarray:
    """``count`` fresh elements of type ``prec`` from ``dist``."""
    return draw_into(rng, prec, empty(prec, count, 0.0), dist, scale)


def draw_integers(rng: np.random.Generator, prec: str, count: int, lo: int, hi: int) -> np.ndarray:
    """Integer-valued elements in [lo, hi] (complex: both parts; double-double:
    lo word zero).  Sums of such values stay exact in every type as long as
    they stay below 2^24 in magnitude."""
    ncomp = 1 if prec in ("s", "d", "w") else 2
    raw = rng.integers(lo, hi + 1, size=count * ncomp).astype(_DTYPE[prec][1])
    if prec in ("s", "d"):
        return raw
    if prec in ("c", "z"):
        return raw.view(_DTYPE[prec][0])
    out = np.zeros((count, 2), dtype=np.float64)
    out[:, 0] = raw
    return out


def place_triangle(prec: str, uplo: str, n: int, lda: int, tri: np.ndarray,
                   fill: float = np.nan) -> np.ndarray:
    """Column-major ``lda x n`` array holding ``tri`` (the stored triangle in
    column-major order) with everything else set to ``fill``."""
    if lda < max(1, n):
        raise ValueError("lda < max(1, n)")
    A = empty(prec, lda * n, fill)
    off = 0
    upper = uplo in ("U", "u")
    for j in range(n):
        r0, r1 = (0, j + 1) if upper else (j, n)
        ln = r1 - r0
        A[j * lda + r0: j * lda + r1] = tri[off: off + ln]
        off += ln
    return A


def diag_index(n: int, lda: int) -> np.ndarray:
    return np.arange(n, dtype=np.int64) * (lda + 1)


@dataclasses.dataclass
class Problem:
    """One call's worth of arguments (host arrays)."""
    prec: str
    uplo: str
    n: int
    lda: int
    alpha: Any
    beta: Any
    A: np.ndarray
    x: np.ndarray
    y: np.ndarray
    incx: int = 1
    incy: int = 1
    name: str = ""

    @property
    def elem_bytes(self) -> int:
        return elem_bytes(self.prec)


def make_problem(prec: str, uplo: str, n: int, lda: int | None = None, *,
                 alpha: Any = 1.0, beta: Any = 1.0, seed: int = 0,
                 a_dist: str = "uniform", xy_dist: str = "uniform",
                 diag_imag_scale: float | None = None,
                 fill: float = np.nan, name: str = "") -> Problem:
    """Draw a problem in the documented order.  ``diag_imag_scale`` (Hermitian
    only) overwrites the imaginary words of the diagonal with uniform values on
    [-scale, scale], drawn last."""
    if prec not in PRECISIONS:
        raise ValueError(prec)
    lda = n if lda is None else lda
    if lda < max(1, n):
        raise ValueError("lda < max(1, n)")
    rng = np.random.Generator(np.random.PCG64(seed))
    # the stored triangle, column by column, drawn straight into place
    A = np.empty((lda * n, 2), dtype=np.float64) if prec == "w" else \
        np.empty(lda * n, dtype=_DTYPE[prec][0])
    fillv = complex(fill, fill) if prec in ("c", "z") else fill
    upper = uplo in ("U", "u")
    for j in range(n):
        r0, r1 = (0, j + 1) if upper else (j, n)
        col = A[j * lda: (j + 1) * lda]
        col[:r0] = fillv
        col[r1:] = fillv
        draw_into(rng, prec, col[r0:r1], a_dist)
    x = draw(rng, prec, n, xy_dist)
    y = draw(rng, prec, n, xy_dist)
    if diag_imag_scale is not None:
        if prec not in ("c", "z"):
            raise ValueError("diagonal garbage only applies to Hermitian types")
        g = draw(rng, "s" if prec == "c" else "d", n, "uniform", diag_imag_scale)
        A.imag[diag_index(n, lda)] = g
    return Problem(prec, uplo, n, lda, alpha, beta, A, x, y, name=name)


def draw_on_device(prec: str, uplo: str, n: int, lda: int | None = None, *,
                   alpha: Any = 1.0, beta: Any = 1.0, seed: int = 0,
                   diag_imag_scale: float | None = None, name: str = "",
                   device=None) -> Problem:
    """The distributions of ``make_problem`` (uniform on [-1, 1]; NaN outside
    the stored triangle; double-double lo = hi*u*2^-53; optional Hermitian
    diagonal garbage) drawn on ``device`` (default: the current CUDA device)
    with torch's seeded generator, for orders whose host draw would take
    minutes.  The
    values differ from ``make_problem``'s for the same seed; the returned
    Problem holds torch device tensors in the host arrays' shapes, and
    ``problem_to_host`` copies it back for the oracle.

    Order of draws: column blocks of A left to right (each block's words,
    then, for double-double, the blocks' u values), then x, then y, then the
    diagonal garbage."""
    import torch
    if prec not in PRECISIONS:
        raise ValueError(prec)
    lda = n if lda is None else lda
    if lda < max(1, n):
        raise ValueError("lda < max(1, n)")
    rdt = torch.float32 if prec in ("s", "c") else torch.float64
    words = 1 if prec in ("s", "d") else 2
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None \
        else torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    upper = uplo in ("U", "u")
    R = torch.empty((n, lda, words), dtype=rdt, device=dev)  # R[j] = column j
    rows = torch.arange(lda, device=dev)
    step = max(1, (1 << 26) // max(1, lda))
    for j0 in range(0, n, step):
        blk = R[j0:j0 + step]
        blk.uniform_(-1.0, 1.0, generator=g)
        if prec == "w":
            u = torch.empty_like(blk[..., 1]).uniform_(-1.0, 1.0, generator=g)
            blk[..., 1] = blk[..., 0] * u * 2.0 ** -53
        cols = torch.arange(j0, j0 + blk.shape[0], device=dev)[:, None]
        outside = (rows[None, :] < cols) if not upper else (rows[None, :] > cols)
        blk.masked_fill_((outside | (rows[None, :] >= n))[..., None], float("nan"))

    def vec():
        v = torch.empty((n, words), dtype=rdt, device=dev).uniform_(-1.0, 1.0, generator=g)
        if prec == "w":
            u = torch.empty(n, dtype=rdt, device=dev).uniform_(-1.0, 1.0, generator=g)
            v[:, 1] = v[:, 0] * u * 2.0 ** -53
        return v

    x, y = vec(), vec()
    if diag_imag_scale is not None:
        if prec not in ("c", "z"):
            raise ValueError("diagonal garbage only applies to Hermitian types")
        d = torch.arange(n, device=dev)
        R[d, d, 1] = torch.empty(n, dtype=rdt, device=dev).uniform_(
            -diag_imag_scale, diag_imag_scale, generator=g)

    def shaped(t, count):
        t = t.reshape(count, words)
        if prec in ("s", "d"):
            return t.reshape(count)
        return torch.view_as_complex(t) if prec in ("c", "z") else t

    return Problem(prec, uplo, n, lda, alpha, beta, shaped(R, lda * n), shaped(x, n),
                   shaped(y, n), name=name)


def gemv_on_device(prec: str, trans: str, m: int, n: int, *, alpha: Any = 1.0,
                   beta: Any = 1.0, seed: int = 0, name: str = "",
                   device=None) -> "GemvProblem":
    """A general m x n product (lda = m) drawn on ``device`` (default: the
    current CUDA device) with torch's seeded generator: A, x and y uniform on
    [-1, 1] (double-double lo = hi*u*2^-53), drawn in that order -- for orders
    whose host draw would take minutes."""
    import torch
    if prec not in PRECISIONS:
        raise ValueError(prec)
    rdt = torch.float32 if prec in ("s", "c") else torch.float64
    words = 1 if prec in ("s", "d") else 2
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None \
        else torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)

    def draw_elems(count):
        t = torch.empty((count, words), dtype=rdt, device=dev).uniform_(-1.0, 1.0, generator=g)
        if prec == "w":
            u = torch.empty(count, dtype=rdt, device=dev).uniform_(-1.0, 1.0, generator=g)
            t[:, 1] = t[:, 0] * u * 2.0 ** -53
        if prec in ("s", "d"):
            return t.reshape(count)
        return torch.view_as_complex(t) if prec in ("c", "z") else t

    lenx, leny = (n, m) if trans in ("N", "n") else (m, n)
    A = draw_elems(m * n)
    x = draw_elems(lenx)
    y = draw_elems(leny)
    return GemvProblem(prec, trans, m, n, m, alpha, beta, A, x, y, name=name)


def problem_to_host(p):
    """A copy of the problem ``p`` (symmetric or general) whose arrays are
    host numpy arrays (device tensors are copied back)."""
    def host(a):
        return a if isinstance(a, np.ndarray) else a.cpu().numpy()
    return dataclasses.replace(p, A=host(p.A), x=host(p.x), y=host(p.y))


CANCEL_SCALE = {"s": 2.0 ** -12, "d": 2.0 ** -30, "c": 2.0 ** -12, "z": 2.0 ** -30,
                "w": 2.0 ** -60}


def make_cancelling_problem(prec: str, uplo: str, n: int, lda: int | None = None, *,
                            seed: int = 0, alpha: Any = 1.0, beta: Any = 0.0,
                            fill: float = np.nan, name: str = "") -> Problem:
    """Heavy cancellation in every row: S = kron(B, [[1, 1], [1, 1]]) + c*E
    (B, E symmetric, Hermitian for complex types, entries uniform on [-1, 1];
    c = CANCEL_SCALE[prec]) and x made of pairs (v, -v), so that row i of S*x
    is about c*(E*x)_i while (|S||x|)_i grows with n.  For double-double the
    hi words hold kron(B, J) and the lo words c*E: every row's hi products
    cancel exactly and the result comes from the lo words alone.  ``n`` must
    be even.

    Draws: B's lower triangle column by column, then E's, then v, then y
    (B, E, v, y as make_problem draws elements; complex values take two
    draws)."""
    if n % 2:
        raise ValueError("n must be even")
    lda = n if lda is None else lda
    rng = np.random.Generator(np.random.PCG64(seed))
    m = n // 2
    cplx = prec in ("c", "z")

    def draw(kind, count):
        return draw_into(rng, kind, empty(kind, count, 0.0))

    def sym(k):
        """Symmetric (Hermitian) k x k matrix from its drawn lower triangle."""
        t = np.zeros((k, k), dtype=np.complex128 if cplx else np.float64)
        for j in range(k):
            col = draw("z" if cplx else "d", k - j)
            t[j:, j] = col
        full = np.tril(t) + np.tril(t, -1).conj().T
        if cplx:
            full[np.diag_indices(k)] = full.diagonal().real
        return full

    B = sym(m)
    E = sym(n)
    J = np.ones((2, 2))
    c = CANCEL_SCALE[prec]
    if prec == "w":
        hi = np.kron(B, J)
        lo = c * E
        dense = np.stack([hi, lo], axis=-1)             # (n, n, 2)
    else:
        dense = (np.kron(B, J) + c * E).astype(_DTYPE[prec][0])
    v = draw(prec, m)
    if prec == "w":
        x = np.empty((n, 2))
        x[0::2] = v
        x[1::2] = -v
    else:
        x = np.empty(n, dtype=_DTYPE[prec][0])
        x[0::2] = v
        x[1::2] = -v
    y = draw(prec, n)
    A = empty(prec, lda * n, fill)
    upper = uplo in ("U", "u")
    for j in range(n):
        r0, r1 = (0, j + 1) if upper else (j, n)
        A[j * lda + r0: j * lda + r1] = dense[r0:r1, j]
    return Problem(prec, uplo, n, lda, alpha, beta, A, x, y, name=name or f"cancel-{prec}{uplo}{n}")


def make_integer_problem(prec: str, uplo: str, n: int, lda: int | None = None, *,
                         alpha: Any = 1.5, beta: Any = -0.5, seed: int = 0,
                         lo: int = -3, hi: int = 3, fill: float = np.nan) -> Problem:
    """Integer-valued A, x, y (entries in [lo, hi]); with alpha = 1.5 and
    beta = -0.5 every intermediate of any summation order is exact while
    n*hi*hi stays below 2^23."""
    lda = n if lda is None else lda
    rng = np.random.Generator(np.random.PCG64(seed))
    tri = draw_integers(rng, prec, n * (n + 1) // 2, lo, hi)
    A = place_triangle(prec, uplo, n, lda, tri, fill)
    x = draw_integers(rng, prec, n, lo, hi)
    y = draw_integers(rng, prec, n, lo, hi)
    if prec == "w":
        alpha = alpha if isinstance(alpha, tuple) else (float(alpha), 0.0)
        beta = beta if isinstance(beta, tuple) else (float(beta), 0.0)
    return Problem(prec, uplo, n, lda, alpha, beta, A, x, y, name="integer")


@dataclasses.dataclass
class GemvProblem:
    """One general matrix-vector call's arguments (host arrays): A is m x n
    column-major with leading dimension lda; x has n elements for trans 'N'
    and m otherwise, y the other length."""
    prec: str
    trans: str
    m: int
    n: int
    lda: int
    alpha: Any
    beta: Any
    A: np.ndarray
    x: np.ndarray
    y: np.ndarray
    incx: int = 1
    incy: int = 1
    name: str = ""

    @property
    def lenx(self) -> int:
        return self.n if self.trans in ("N", "n") else self.m

    @property
    def leny(self) -> int:
        return self.m if self.trans in ("N", "n") else self.n


def make_gemv_problem(prec: str, trans: str, m: int, n: int, lda: int | None = None, *,
                      alpha: Any = 1.0, beta: Any = 1.0, seed: int = 0,
                      a_dist: str = "uniform", xy_dist: str = "uniform",
                      fill: float = np.nan, integer: tuple[int, int] | None = None,
                      name: str = "") -> GemvProblem:
    """Draw a general problem: A column by column (rows 0..m-1; padding rows
    hold `fill`), then x, then y.  ``integer = (lo, hi)`` draws integers
    instead."""
    if prec not in PRECISIONS:
        raise ValueError(prec)
    lda = m if lda is None else lda
    if lda < max(1, m):
        raise ValueError("lda < max(1, m)")
    rng = np.random.Generator(np.random.PCG64(seed))
    A = np.empty((lda * n, 2), dtype=np.float64) if prec == "w" else \
        np.empty(lda * n, dtype=_DTYPE[prec][0])
    fillv = complex(fill, fill) if prec in ("c", "z") else fill
    for j in range(n):
        col = A[j * lda: (j + 1) * lda]
        col[m:] = fillv
        if integer is None:
            draw_into(rng, prec, col[:m], a_dist)
        else:
            col[:m] = draw_integers(rng, prec, m, *integer)
    lx, ly = (n, m) if trans in ("N", "n") else (m, n)
    if integer is None:
        x = draw(rng, prec, lx, xy_dist)
        y = draw(rng, prec, ly, xy_dist)
    else:
        x = draw_integers(rng, prec, lx, *integer)
        y = draw_integers(rng, prec, ly, *integer)
        if prec == "w":
            alpha = alpha if isinstance(alpha, tuple) else (float(alpha), 0.0)
            beta = beta if isinstance(beta, tuple) else (float(beta), 0.0)
    return GemvProblem(prec, trans, m, n, lda, alpha, beta, A, x, y, name=name)


@dataclasses.dataclass
class Syr2Problem:
    """One rank-2 update's arguments (host arrays): A holds the stored
    triangle (the other triangle and padding hold `fill`)."""
    prec: str
    uplo: str
    n: int
    lda: int
    alpha: Any
    x: np.ndarray
    y: np.ndarray
    A: np.ndarray
    incx: int = 1
    incy: int = 1
    name: str = ""


def make_syr2_problem(prec: str, uplo: str, n: int, lda: int | None = None, *,
                      alpha: Any = 1.0, seed: int = 0, fill: float = np.nan,
                      diag_imag_scale: float | None = None,
                      integer: tuple[int, int] | None = None, name: str = "") -> Syr2Problem:
    """Draw a rank-2 update: the stored triangle column by column (as
    make_problem does), then x, then y, then (Hermitian) the diagonal's
    imaginary words, which the update must overwrite with zero."""
    if integer is None:
        p = make_problem(prec, uplo, n, lda, alpha=alpha, beta=alpha, seed=seed, fill=fill,
                         diag_imag_scale=diag_imag_scale)
        return Syr2Problem(prec, uplo, n, p.lda, alpha, p.x, p.y, p.A, name=name)
    p = make_integer_problem(prec, uplo, n, lda, alpha=alpha, beta=alpha, seed=seed,
                             lo=integer[0], hi=integer[1], fill=fill)
    return Syr2Problem(prec, uplo, n, p.lda, p.alpha, p.x, p.y, p.A, name=name)


@dataclasses.dataclass
class TrmvProblem:
    """One triangular product's arguments (host arrays): A holds the stored
    triangle (diagonal included; the other triangle and padding hold `fill`)."""
    prec: str
    uplo: str
    trans: str
    diag: str
    n: int
    lda: int
    A: np.ndarray
    x: np.ndarray
    incx: int = 1
    name: str = ""


def make_trmv_problem(prec: str, uplo: str, trans: str, diag: str, n: int,
                      lda: int | None = None, *, seed: int = 0, fill: float = np.nan,
                      integer: tuple[int, int] | None = None,
                      name: str = "") -> TrmvProblem:
    """Draw a triangular product: the stored triangle column by column (as
    make_problem does), then x (the same draws as a symmetric problem's)."""
    if integer is None:
        p = make_problem(prec, uplo, n, lda, seed=seed, fill=fill)
    else:
        p = make_integer_problem(prec, uplo, n, lda, seed=seed, lo=integer[0], hi=integer[1],
                                 fill=fill)
    return TrmvProblem(prec, uplo, trans, diag, n, p.lda, p.A, p.x, name=name)


# --------------------------------------------------------------------------
# The benchmark workloads, named by what they are.
# --------------------------------------------------------------------------

SWEEP_N = (2048, 4096, 8192, 16384, 24576, 32768, 10007, 32767)


def ssymv_lower_n1024() -> Problem:
    """SSYMV, uplo=L, n=lda=1024, uniform A, x, y; alpha=1.5, beta=-0.5; seed 0."""
    return make_problem("s", "L", 1024, 1024, alpha=1.5, beta=-0.5, seed=0,
                        name="ssymv-L-n1024")


def dsymv_upper_n8192_lda8200_beta0() -> Problem:
    """DSYMV, uplo=U, n=8192, lda=8200, uniform A, normal x, y; alpha=1,
    beta=0 (y is ignored); seed 1."""
    return make_problem("d", "U", 8192, 8200, alpha=1.0, beta=0.0, seed=1,
                        xy_dist="normal", name="dsymv-U-n8192-lda8200-beta0")


def symv_sweep(prec: str, uplo: str, n: int) -> Problem:
    """[SD]SYMV size sweep: lda=n, uniform A, x, y; alpha=beta=1; seed=n."""
    if prec not in ("s", "d"):
        raise ValueError(prec)
    return make_problem(prec, uplo, n, n, alpha=1.0, beta=1.0, seed=n,
                        name=f"{prec}symv-{uplo}-n{n}")


def hemv_lower_n16384(prec: str, n: int = 16384) -> Problem:
    """[CZ]HEMV, uplo=L, n=16384, uniform A, x, y, diagonal imaginary words
    uniform[-1e3, 1e3] (must be ignored); alpha=(0.75,0.25), beta=(0.5,-1);
    seed 3."""
    if prec not in ("c", "z"):
        raise ValueError(prec)
    return make_problem(prec, "L", n, n, alpha=complex(0.75, 0.25),
                        beta=complex(0.5, -1.0), seed=3, diag_imag_scale=1e3,
                        name=f"{prec}hemv-L-n{n}")


def wsymv_lower_n8192(n: int = 8192) -> Problem:
    """WSYMV (double-double), uplo=L, n=8192, (hi, lo) with hi uniform[-1,1]
    and lo = hi*u*2^-53; alpha = beta = (1, 0); seed 4."""
    return make_problem("w", "L", n, n, alpha=(1.0, 0.0), beta=(1.0, 0.0),
                        seed=4, name=f"wsymv-L-n{n}")


def metric_order_on_device(prec: str, n: int = 32768, uplo: str = "L") -> Problem:
    """lda = n, seed n, drawn on the device: [SD]SYMV with alpha = beta = 1;
    [CZ]HEMV with the n = 16384 workload's scalars and diagonal garbage;
    WSYMV with alpha = beta = (1, 0)."""
    kw = {"s": dict(alpha=1.0, beta=1.0), "d": dict(alpha=1.0, beta=1.0),
          "c": dict(alpha=complex(0.75, 0.25), beta=complex(0.5, -1.0), diag_imag_scale=1e3),
          "z": dict(alpha=complex(0.75, 0.25), beta=complex(0.5, -1.0), diag_imag_scale=1e3),
          "w": dict(alpha=(1.0, 0.0), beta=(1.0, 0.0))}[prec]
    kind = "hemv" if prec in ("c", "z") else "symv"
    return draw_on_device(prec, uplo, n, n, seed=n, name=f"{prec}{kind}-{uplo}-n{n}-devdraw", **kw)


def gemv_square(prec: str, trans: str, n: int) -> GemvProblem:
    """xGEMV beside the [SD]SYMV sweep: m = n = lda, uniform A, x, y;
    alpha = beta = 1; seed = n."""
    return make_gemv_problem(prec, trans, n, n, n, alpha=1.0, beta=1.0, seed=n,
                             name=f"{prec}gemv-{trans}-n{n}")
