"""Native test checkers, compiled with gcc on first use."""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_BUILD = os.path.join(_HERE, "_build")
_lib = None


def quad_lib():
    global _lib
    if _lib is None:
        os.makedirs(_BUILD, exist_ok=True)
        so = os.path.join(_BUILD, "libquadref.so")
        tmp = so + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-std=gnu99", "-fPIC", "-shared", "-o", tmp,
                        os.path.join(_HERE, "quadref.c"), "-lquadmath"],
                       check=True)
        os.replace(tmp, so)
        lib = ctypes.CDLL(so)
        vp, ci = ctypes.c_void_p, ctypes.c_int
        for nm in ("quad_wsymv_rows", "quad_dsymv_rows"):
            f = getattr(lib, nm)
            f.restype = ci
            f.argtypes = [ctypes.c_char, ci, vp, vp, ci, vp, vp, vp, vp, ci, vp, vp]
        for nm in ("quad_wgemv_rows", "quad_dgemv_rows"):
            f = getattr(lib, nm)
            f.restype = ci
            f.argtypes = [ctypes.c_char, ci, ci, vp, vp, ci, vp, vp, vp, vp, ci, vp, vp]
        _lib = lib
    return _lib


def quad_rows(p, rows):
    """binary128 rows of alpha*S*x + beta*y for a 'w' or 'd' problem with unit
    increments; returns an (nrows, 2) float64 array of (hi, lo)."""
    assert p.incx == 1 and p.incy == 1
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    hi = np.empty(len(rows))
    lo = np.empty(len(rows))
    if p.prec == "w":
        al = np.array(p.alpha, dtype=np.float64)
        be = np.array(p.beta, dtype=np.float64)
        f = quad_lib().quad_wsymv_rows
    else:
        al = np.array([p.alpha], dtype=np.float64)
        be = np.array([p.beta], dtype=np.float64)
        f = quad_lib().quad_dsymv_rows
    A = np.ascontiguousarray(p.A)
    x = np.ascontiguousarray(p.x)
    y = np.ascontiguousarray(p.y)
    rc = f(p.uplo.encode(), p.n, al.ctypes.data, A.ctypes.data, p.lda,
           x.ctypes.data, be.ctypes.data, y.ctypes.data, rows.ctypes.data,
           len(rows), hi.ctypes.data, lo.ctypes.data)
    assert rc == 0
    return np.stack([hi, lo], axis=1)


def quad_gemv_rows(p, rows):
    """binary128 output elements ``rows`` of alpha*op(A)*x + beta*y for a 'w'
    or 'd' GemvProblem with unit increments; (nrows, 2) float64 (hi, lo)."""
    assert p.incx == 1 and p.incy == 1
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    hi = np.empty(len(rows))
    lo = np.empty(len(rows))
    if p.prec == "w":
        al = np.array(p.alpha, dtype=np.float64)
        be = np.array(p.beta, dtype=np.float64)
        f = quad_lib().quad_wgemv_rows
    else:
        al = np.array([p.alpha], dtype=np.float64)
        be = np.array([p.beta], dtype=np.float64)
        f = quad_lib().quad_dgemv_rows
    A = np.ascontiguousarray(p.A)
    x = np.ascontiguousarray(p.x)
    y = np.ascontiguousarray(p.y)
    rc = f(p.trans.encode(), p.m, p.n, al.ctypes.data, A.ctypes.data, p.lda,
           x.ctypes.data, be.ctypes.data, y.ctypes.data, rows.ctypes.data,
           len(rows), hi.ctypes.data, lo.ctypes.data)
    assert rc == 0
    return np.stack([hi, lo], axis=1)


ABI_CALLER = os.path.join(_HERE, "bin", "abi_caller")


def build_abi_caller() -> str:
    """Compile the plain host program that calls libxsymv through its C header
    (hipcc, host code only); libxsymv and the oracle library must be built."""
    root = os.path.dirname(os.path.dirname(_HERE))
    os.makedirs(os.path.dirname(ABI_CALLER), exist_ok=True)
    tmp = ABI_CALLER + f".tmp{os.getpid()}"
    lib_dir = os.path.join(root, "blas_symmetric_mat_amd")
    ora_dir = os.path.join(root, "oracle")
    subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-std=c++17", "-o", tmp,
                    os.path.join(_HERE, "abi_caller.cpp"),
                    "-I", os.path.join(root, "include"), "-I", ora_dir,
                    "-L", lib_dir, "-lxsymv", "-L", ora_dir, "-loracle_xsymv",
                    "-Wl,-rpath,$ORIGIN/../../../blas_symmetric_mat_amd:$ORIGIN/../../../oracle"],
                   check=True)
    os.replace(tmp, ABI_CALLER)
    return ABI_CALLER
