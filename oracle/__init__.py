"""ctypes binding of the CPU oracle (``xsymv_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only the tests, the packaged smoke check and the
benchmark's CPU-baseline leg may import this module.  It never imports the
GPU package, and the GPU package never imports it.

Arrays are numpy arrays in the element storage documented in
``blas_symmetric_mat_amd.workloads`` (float32, float64, complex64,
complex128, or float64 with a trailing axis of 2 for double-double).
Scalars: float for 's'/'d', complex for 'c'/'z', (hi, lo) for 'w'.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "xsymv_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle_xsymv.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-std=c99", "-fPIC", "-shared", "-Wall", "-fopenmp"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``liboracle_xsymv.so``."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True,
                   cwd=_HERE)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _CF(ctypes.Structure):
    _fields_ = [("re", ctypes.c_float), ("im", ctypes.c_float)]


class _CD(ctypes.Structure):
    _fields_ = [("re", ctypes.c_double), ("im", ctypes.c_double)]


class _DD(ctypes.Structure):
    _fields_ = [("hi", ctypes.c_double), ("lo", ctypes.c_double)]


_SCALAR = {"s": ctypes.c_float, "d": ctypes.c_double, "c": _CF, "z": _CD, "w": _DD}
_NAME = {"s": "ssymv", "d": "dsymv", "c": "chemv", "z": "zhemv", "w": "wsymv"}
_GNAME = {"s": "sgemv", "d": "dgemv", "c": "cgemv", "z": "zgemv", "w": "wgemv"}
_RNAME = {"s": "ssyr2", "d": "dsyr2", "c": "cher2", "z": "zher2", "w": "wsyr2"}
_TNAME = {"s": "strmv", "d": "dtrmv", "c": "ctrmv", "z": "ztrmv", "w": "wtrmv"}
_SHNAME = {"s": "ssymv_shard", "d": "dsymv_shard", "c": "chemv_shard", "z": "zhemv_shard",
           "w": "wsymv_shard"}
_NP = {"s": np.float32, "d": np.float64, "c": np.complex64, "z": np.complex128,
       "w": np.float64}

def _declare(lib):
    vp = ctypes.c_void_p
    ci = ctypes.c_int
    for p, nm in _NAME.items():
        st = _SCALAR[p]
        f = getattr(lib, "oracle_" + nm)
        f.restype = ci
        f.argtypes = [ctypes.c_char, ci, st, vp, ci, vp, ci, st, vp, ci]
        g = getattr(lib, "oracle_" + nm + "_rows")
        g.restype = ci
        g.argtypes = [ctypes.c_char, ci, st, vp, ci, vp, ci, st, vp, ci,
                      vp, ci, vp]
    for p, nm in _GNAME.items():
        st = _SCALAR[p]
        f = getattr(lib, "oracle_" + nm)
        f.restype = ci
        f.argtypes = [ctypes.c_char, ci, ci, st, vp, ci, vp, ci, st, vp, ci]
        g = getattr(lib, "oracle_" + nm + "_rows")
        g.restype = ci
        g.argtypes = [ctypes.c_char, ci, ci, st, vp, ci, vp, ci, st, vp, ci,
                      vp, ci, vp]
    for p, nm in _RNAME.items():
        f = getattr(lib, "oracle_" + nm)
        f.restype = ci
        f.argtypes = [ctypes.c_char, ci, _SCALAR[p], vp, ci, vp, ci, vp, ci]
    for p, nm in _TNAME.items():
        f = getattr(lib, "oracle_" + nm)
        f.restype = ci
        f.argtypes = [ctypes.c_char, ctypes.c_char, ctypes.c_char, ci, vp, ci, vp, ci]
    for p, nm in _SHNAME.items():
        f = getattr(lib, "oracle_" + nm)
        f.restype = ci
        f.argtypes = [ctypes.c_char, ci, ci, ci, ci, vp, ci, vp, ci, vp]
        f = getattr(lib, f"oracle_{p}combine")
        f.restype = ci
        f.argtypes = [ci, ci, _SCALAR[p], vp, ci, _SCALAR[p], vp, ci]
    lib.oracle_set_threads.restype = ci
    lib.oracle_set_threads.argtypes = [ci]
    lib.oracle_get_threads.restype = ci
    lib.oracle_get_threads.argtypes = []
    lib.oracle_shard_columns.restype = ci
    lib.oracle_shard_columns.argtypes = [ci, ci, ci, ci, vp]
    for nm in ("oracle_dd_add", "oracle_dd_mul"):
        f = getattr(lib, nm)
        f.restype = _DD
        f.argtypes = [_DD, _DD]
    return lib


def scalar(prec: str, value):
    """ctypes scalar of type ``prec`` from a Python value."""
    if prec in ("s", "d"):
        return _SCALAR[prec](float(value))
    if prec in ("c", "z"):
        v = complex(value)
        return _SCALAR[prec](v.real, v.imag)
    hi, lo = value
    return _DD(float(hi), float(lo))


def _ptr(a):
    if a is None:
        return None
    if not isinstance(a, np.ndarray):
        raise TypeError("numpy array expected")
    if not a.flags.c_contiguous:
        raise ValueError("array must be contiguous")
    return a.ctypes.data


def _check_dtype(prec, *arrays):
    for a in arrays:
        if a is not None and a.dtype != _NP[prec]:
            raise TypeError(f"dtype {a.dtype} does not match precision {prec!r}")


def _uplo(uplo):
    return uplo.encode()[:1] if isinstance(uplo, str) else uplo


class OracleLib:
    """The oracle loaded from one shared-library file."""

    def __init__(self, path: str):
        self.path = path
        self._lib = _declare(ctypes.CDLL(path))

    def symv(self, prec: str, uplo: str, n: int, alpha, A, lda: int, x,
             incx: int, beta, y, incy: int) -> int:
        """y := alpha*S*x + beta*y in place, from the definition (one
        output at a time, inner index ascending).
        Returns the status code (0 = ok, negative = bad argument)."""
        _check_dtype(prec, A, x, y)
        f = getattr(self._lib, "oracle_" + _NAME[prec])
        return f(_uplo(uplo), n, scalar(prec, alpha), _ptr(A), lda, _ptr(x),
                 incx, scalar(prec, beta), _ptr(y), incy)

    def symv_rows(self, prec: str, uplo: str, n: int, alpha, A, lda: int, x,
                  incx: int, beta, y, incy: int, rows) -> np.ndarray:
        """Rows ``rows`` of alpha*S*x + beta*y from the definition (y is not
        modified)."""
        _check_dtype(prec, A, x, y)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        shape = (len(rows), 2) if prec == "w" else (len(rows),)
        out = np.empty(shape, dtype=_NP[prec])
        f = getattr(self._lib, "oracle_" + _NAME[prec] + "_rows")
        rc = f(_uplo(uplo), n, scalar(prec, alpha), _ptr(A), lda, _ptr(x),
               incx, scalar(prec, beta), _ptr(y), incy, _ptr(rows), len(rows),
               _ptr(out))
        if rc != 0:
            raise ValueError(f"oracle rows call failed with status {rc}")
        return out

    def symv_problem(self, p, y=None):
        """Run on a ``workloads.Problem``; returns the new y (a copy)."""
        y = (p.y if y is None else y).copy()
        rc = self.symv(p.prec, p.uplo, p.n, p.alpha, p.A, p.lda, p.x, p.incx,
                       p.beta, y, p.incy)
        if rc != 0:
            raise ValueError(f"oracle call failed with status {rc}")
        return y

    def rows_problem(self, p, rows=None):
        rows = np.arange(p.n) if rows is None else rows
        return self.symv_rows(p.prec, p.uplo, p.n, p.alpha, p.A, p.lda, p.x,
                              p.incx, p.beta, p.y, p.incy, rows)

    def gemv(self, prec: str, trans: str, m: int, n: int, alpha, A, lda: int, x,
             incx: int, beta, y, incy: int) -> int:
        """y := alpha*op(A)*x + beta*y in place, from the definition.
        Returns the status code (0 = ok, negative = bad argument)."""
        _check_dtype(prec, A, x, y)
        f = getattr(self._lib, "oracle_" + _GNAME[prec])
        return f(_uplo(trans), m, n, scalar(prec, alpha), _ptr(A), lda, _ptr(x),
                 incx, scalar(prec, beta), _ptr(y), incy)

    def gemv_rows(self, prec: str, trans: str, m: int, n: int, alpha, A, lda: int,
                  x, incx: int, beta, y, incy: int, rows) -> np.ndarray:
        """Output elements ``rows`` of alpha*op(A)*x + beta*y (y not modified)."""
        _check_dtype(prec, A, x, y)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        shape = (len(rows), 2) if prec == "w" else (len(rows),)
        out = np.empty(shape, dtype=_NP[prec])
        f = getattr(self._lib, "oracle_" + _GNAME[prec] + "_rows")
        rc = f(_uplo(trans), m, n, scalar(prec, alpha), _ptr(A), lda, _ptr(x),
               incx, scalar(prec, beta), _ptr(y), incy, _ptr(rows), len(rows),
               _ptr(out))
        if rc != 0:
            raise ValueError(f"oracle gemv rows call failed with status {rc}")
        return out

    def gemv_problem(self, p, y=None):
        """Run on a ``workloads.GemvProblem``; returns the new y (a copy)."""
        y = (p.y if y is None else y).copy()
        rc = self.gemv(p.prec, p.trans, p.m, p.n, p.alpha, p.A, p.lda, p.x, p.incx,
                       p.beta, y, p.incy)
        if rc != 0:
            raise ValueError(f"oracle gemv call failed with status {rc}")
        return y

    def gemv_rows_problem(self, p, rows=None):
        rows = np.arange(p.leny) if rows is None else rows
        return self.gemv_rows(p.prec, p.trans, p.m, p.n, p.alpha, p.A, p.lda, p.x,
                              p.incx, p.beta, p.y, p.incy, rows)

    def syr2(self, prec: str, uplo: str, n: int, alpha, x, incx: int, y, incy: int, A,
             lda: int) -> int:
        """A := alpha*x*y^H + conj(alpha)*y*x^H + A on the stored triangle, in
        place.  Returns the status code."""
        _check_dtype(prec, A, x, y)
        f = getattr(self._lib, "oracle_" + _RNAME[prec])
        return f(_uplo(uplo), n, scalar(prec, alpha), _ptr(x), incx, _ptr(y), incy,
                 _ptr(A), lda)

    def syr2_problem(self, p, A=None):
        """Run on a ``workloads.Syr2Problem``; returns the new A (a copy)."""
        A = (p.A if A is None else A).copy()
        rc = self.syr2(p.prec, p.uplo, p.n, p.alpha, p.x, p.incx, p.y, p.incy, A, p.lda)
        if rc != 0:
            raise ValueError(f"oracle syr2 call failed with status {rc}")
        return A

    def trmv(self, prec: str, uplo: str, trans: str, diag: str, n: int, A, lda: int, x,
             incx: int) -> int:
        """x := op(T)*x in place; returns the status code."""
        _check_dtype(prec, A, x)
        f = getattr(self._lib, "oracle_" + _TNAME[prec])
        return f(_uplo(uplo), _uplo(trans), _uplo(diag), n, _ptr(A), lda, _ptr(x), incx)

    def trmv_problem(self, p, x=None):
        """Run on a ``workloads.TrmvProblem``; returns the new x (a copy)."""
        x = (p.x if x is None else x).copy()
        rc = self.trmv(p.prec, p.uplo, p.trans, p.diag, p.n, p.A, p.lda, x, p.incx)
        if rc != 0:
            raise ValueError(f"oracle trmv call failed with status {rc}")
        return x

    def shard_columns(self, n: int, panel: int, nshards: int, shard: int) -> np.ndarray:
        """The shard's global columns, ascending."""
        k = self._lib.oracle_shard_columns(n, panel, nshards, shard, None)
        if k < 0:
            raise ValueError("bad shard arguments")
        cols = np.zeros(max(k, 1), dtype=np.int32)
        self._lib.oracle_shard_columns(n, panel, nshards, shard, _ptr(cols))
        return cols[:k]

    def shard(self, prec: str, uplo: str, n: int, panel: int, nshards: int, shard: int, Aloc,
              lda: int, x, incx: int, p) -> int:
        """p := the shard's partial product (n elements, contiguous); returns
        the status code."""
        _check_dtype(prec, Aloc, x, p)
        f = getattr(self._lib, "oracle_" + _SHNAME[prec])
        return f(_uplo(uplo), n, panel, nshards, shard, _ptr(Aloc), lda, _ptr(x), incx, _ptr(p))

    def combine(self, prec: str, n: int, nshards: int, alpha, P, ldp: int, beta, y,
                incy: int) -> int:
        """y := beta*y + alpha*(P_0 + P_1 + ...) in place; returns the status."""
        _check_dtype(prec, P, y)
        f = getattr(self._lib, f"oracle_{prec}combine")
        return f(n, nshards, scalar(prec, alpha), _ptr(P), ldp, scalar(prec, beta), _ptr(y),
                 incy)

    def set_threads(self, nthreads: int) -> int:
        """Threads of the full-product calls (outputs are independent, so
        every count gives the same bits); returns 0 or a negative code."""
        return self._lib.oracle_set_threads(int(nthreads))

    def get_threads(self) -> int:
        return self._lib.oracle_get_threads()

    def dd_add(self, a, b):
        r = self._lib.oracle_dd_add(_DD(*a), _DD(*b))
        return (r.hi, r.lo)

    def dd_mul(self, a, b):
        r = self._lib.oracle_dd_mul(_DD(*a), _DD(*b))
        return (r.hi, r.lo)


_default = None
_lock = threading.Lock()


def default() -> OracleLib:
    """The oracle built from this directory's source (built on first use)."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(LIB_PATH):
                build()
            _default = OracleLib(LIB_PATH)
    return _default


def symv(*a, **k):
    return default().symv(*a, **k)


def symv_rows(*a, **k):
    return default().symv_rows(*a, **k)


def symv_problem(p, y=None):
    return default().symv_problem(p, y)


def rows_problem(p, rows=None):
    return default().rows_problem(p, rows)


def dd_add(a, b):
    return default().dd_add(a, b)


def set_threads(nthreads):
    return default().set_threads(nthreads)


def get_threads():
    return default().get_threads()


def dd_mul(a, b):
    return default().dd_mul(a, b)


def gemv(*a, **k):
    return default().gemv(*a, **k)


def gemv_rows(*a, **k):
    return default().gemv_rows(*a, **k)


def gemv_problem(p, y=None):
    return default().gemv_problem(p, y)


def gemv_rows_problem(p, rows=None):
    return default().gemv_rows_problem(p, rows)


def syr2(*a, **k):
    return default().syr2(*a, **k)


def syr2_problem(p, A=None):
    return default().syr2_problem(p, A)


def trmv(*a, **k):
    return default().trmv(*a, **k)


def trmv_problem(p, x=None):
    return default().trmv_problem(p, x)


def shard_columns(*a, **k):
    return default().shard_columns(*a, **k)


def shard(*a, **k):
    return default().shard(*a, **k)


def combine(*a, **k):
    return default().combine(*a, **k)
