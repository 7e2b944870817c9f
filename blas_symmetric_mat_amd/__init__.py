"""Python binding of libxsymv (MI355X / gfx950 SYMV, HEMV and WSYMV).

Argument marshalling only: every step of the product runs in the library's
HIP kernels.  The names and argument lists are those of the C ABI
(``include/xsymv.h``): ``xsymv_s``, ``xsymv_d``, ``xhemv_c``, ``xhemv_z``,
``xsymv_w`` compute y := alpha*S*x + beta*y from one stored triangle.

Device arrays may be passed as torch tensors (their ``data_ptr()``) or as
integer device addresses.  ``stream`` defaults to torch's current HIP stream
on the current device.  A non-zero status raises ``XsymvError``.

There is no fallback: if ``libxsymv.so`` has not been built, the first call
raises ``ImportError``.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = ["xsymv_s", "xsymv_d", "xhemv_c", "xhemv_z", "xsymv_w", "XsymvError",
           "library", "LIB_PATH", "PREC_CODE", "workspace_bytes", "num_configs",
           "config_info", "select_config", "current_config", "timing_enable",
           "timing_read", "release", "version"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libxsymv.so")
PREC_CODE = {"s": 0, "d": 1, "c": 2, "z": 3, "w": 4}


class XsymvError(RuntimeError):
    def __init__(self, name, code):
        self.code = code
        if code >= 1000:
            msg = f"{name}: HIP runtime error {code - 1000}"
        else:
            msg = f"{name}: illegal value of argument {-code}"
        super().__init__(msg)


class _C64(ctypes.Structure):
    _fields_ = [("re", ctypes.c_float), ("im", ctypes.c_float)]


class _C128(ctypes.Structure):
    _fields_ = [("re", ctypes.c_double), ("im", ctypes.c_double)]


class _DD(ctypes.Structure):
    _fields_ = [("hi", ctypes.c_double), ("lo", ctypes.c_double)]


_SCALAR = {"s": ctypes.c_float, "d": ctypes.c_double, "c": _C64, "z": _C128, "w": _DD}
_ENTRY = {"s": "xsymv_s", "d": "xsymv_d", "c": "xhemv_c", "z": "xhemv_z", "w": "xsymv_w"}

_lib = None
_lock = threading.Lock()


def library():
    """The loaded ``libxsymv.so`` (ctypes), with argument types declared."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m blas_symmetric_mat_amd.build` (hipcc, gfx950)")
            lib = ctypes.CDLL(LIB_PATH)
            vp, ci, cc = ctypes.c_void_p, ctypes.c_int, ctypes.c_char
            for p, nm in _ENTRY.items():
                f = getattr(lib, nm)
                st = _SCALAR[p]
                f.restype = ci
                f.argtypes = [cc, ci, st, vp, ci, vp, ci, st, vp, ci, vp]
            lib.xsymv_workspace_bytes.restype = ctypes.c_size_t
            lib.xsymv_workspace_bytes.argtypes = [ci, cc, ci]
            lib.xsymv_release.restype = ci
            lib.xsymv_release.argtypes = []
            lib.xsymv_num_configs.restype = ci
            lib.xsymv_num_configs.argtypes = [ci]
            ip = ctypes.POINTER(ci)
            lib.xsymv_config_info.restype = ci
            lib.xsymv_config_info.argtypes = [ci, ci, ip, ip, ip, ip, ip]
            lib.xsymv_select_config.restype = ci
            lib.xsymv_select_config.argtypes = [ci, cc, ci, ci, ci]
            lib.xsymv_current_config.restype = ci
            lib.xsymv_current_config.argtypes = [ci, cc, ci]
            lib.xsymv_timing_enable.restype = ci
            lib.xsymv_timing_enable.argtypes = [ci]
            fp = ctypes.POINTER(ctypes.c_float)
            lib.xsymv_timing_read.restype = ci
            lib.xsymv_timing_read.argtypes = [fp, fp, ci]
            lib.xsymv_version.restype = ctypes.c_char_p
            lib.xsymv_version.argtypes = []
            _lib = lib
    return _lib


def _scalar(prec, v):
    if prec in ("s", "d"):
        return _SCALAR[prec](float(v))
    if prec in ("c", "z"):
        v = complex(v)
        return _SCALAR[prec](v.real, v.imag)
    hi, lo = v
    return _DD(float(hi), float(lo))


def _addr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(prec, uplo, n, alpha, A, lda, x, incx, beta, y, incy, stream):
    f = getattr(library(), _ENTRY[prec])
    u = uplo.encode()[:1] if isinstance(uplo, str) else uplo
    rc = f(u, n, _scalar(prec, alpha), _addr(A), lda, _addr(x), incx,
           _scalar(prec, beta), _addr(y), incy, _stream(stream))
    if rc != 0:
        raise XsymvError(_ENTRY[prec], rc)


def xsymv_s(uplo, n, alpha, A, lda, x, incx, beta, y, incy, stream=None):
    """SSYMV: y := alpha*S*x + beta*y, float32, S symmetric (one triangle)."""
    _call("s", uplo, n, alpha, A, lda, x, incx, beta, y, incy, stream)


def xsymv_d(uplo, n, alpha, A, lda, x, incx, beta, y, incy, stream=None):
    """DSYMV: y := alpha*S*x + beta*y, float64, S symmetric (one triangle)."""
    _call("d", uplo, n, alpha, A, lda, x, incx, beta, y, incy, stream)


def xhemv_c(uplo, n, alpha, A, lda, x, incx, beta, y, incy, stream=None):
    """CHEMV: complex64, S Hermitian (one triangle; diagonal imaginary words
    ignored)."""
    _call("c", uplo, n, alpha, A, lda, x, incx, beta, y, incy, stream)


def xhemv_z(uplo, n, alpha, A, lda, x, incx, beta, y, incy, stream=None):
    """ZHEMV: complex128, S Hermitian."""
    _call("z", uplo, n, alpha, A, lda, x, incx, beta, y, incy, stream)


def xsymv_w(uplo, n, alpha, A, lda, x, incx, beta, y, incy, stream=None):
    """WSYMV: double-double (hi, lo pairs); alpha, beta are (hi, lo) tuples."""
    _call("w", uplo, n, alpha, A, lda, x, incx, beta, y, incy, stream)


def workspace_bytes(prec: str, uplo: str, n: int) -> int:
    return library().xsymv_workspace_bytes(PREC_CODE[prec], uplo.encode()[:1], n)


def num_configs(prec: str) -> int:
    return library().xsymv_num_configs(PREC_CODE[prec])


def config_info(prec: str, idx: int) -> dict:
    vals = [ctypes.c_int() for _ in range(5)]
    rc = library().xsymv_config_info(PREC_CODE[prec], idx, *[ctypes.byref(v) for v in vals])
    if rc != 0:
        raise IndexError(idx)
    w, cw, s, h, nt = (v.value for v in vals)
    return {"waves": w, "cols_per_wave": cw, "stripes": s, "rows_per_stripe": h,
            "nontemporal": nt, "panel": w * cw, "tile_rows": s * h}


def select_config(prec: str, uplo: str, n_lo: int, n_hi: int, idx: int) -> None:
    rc = library().xsymv_select_config(PREC_CODE[prec], uplo.encode()[:1], n_lo, n_hi, idx)
    if rc != 0:
        raise ValueError("bad configuration selection")


def current_config(prec: str, uplo: str, n: int) -> int:
    return library().xsymv_current_config(PREC_CODE[prec], uplo.encode()[:1], n)


def timing_enable(on: bool) -> None:
    library().xsymv_timing_enable(1 if on else 0)


def timing_read(max_calls: int = 4096):
    """List of (main_kernel_ms, merge_kernel_ms) for the calls recorded since
    timing was enabled or last read."""
    a = (ctypes.c_float * max_calls)()
    b = (ctypes.c_float * max_calls)()
    k = library().xsymv_timing_read(a, b, max_calls)
    if k >= 1000:
        raise XsymvError("xsymv_timing_read", k)
    return [(a[i], b[i]) for i in range(k)]


def release() -> None:
    rc = library().xsymv_release()
    if rc != 0:
        raise XsymvError("xsymv_release", rc)


def version() -> str:
    return library().xsymv_version().decode()
