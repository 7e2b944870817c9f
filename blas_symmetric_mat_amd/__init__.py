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
           "timing_read", "release", "version", "autotune", "save_config", "load_config",
           "clear_config", "strip_plan", "config_workgroups", "set_workspace", "read_bandwidth",
           "xgemv_s", "xgemv_d", "xgemv_c", "xgemv_z", "xgemv_w", "gemv_num_configs",
           "gemv_config_info", "gemv_select_config", "gemv_current_config",
           "gemv_workspace_bytes", "gemv_plan", "xsyr2_s", "xsyr2_d", "xher2_c", "xher2_z",
           "xsyr2_w", "syr2_num_configs", "syr2_config_info", "syr2_select_config",
           "syr2_current_config", "xtrmv_s", "xtrmv_d", "xtrmv_c", "xtrmv_z", "xtrmv_w",
           "trmv_num_configs", "trmv_config_info", "trmv_select_config", "trmv_current_config",
           "trmv_workspace_bytes", "xsymv_shard_s", "xsymv_shard_d", "xhemv_shard_c",
           "xhemv_shard_z", "xsymv_shard_w", "xsymv_combine_s", "xsymv_combine_d",
           "xhemv_combine_c", "xhemv_combine_z", "xsymv_combine_w", "shard_columns", "shard_plan",
           "shard_workspace_bytes", "copy_bandwidth", "xsymv_s_noalloc", "STATIC_SCRATCH_BYTES"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libxsymv.so")
PREC_CODE = {"s": 0, "d": 1, "c": 2, "z": 3, "w": 4}
# XSYMV_STATIC_SCRATCH_BYTES of include/xsymv.h: the static array of xsymv_s_noalloc
STATIC_SCRATCH_BYTES = 32 << 20


class XsymvError(RuntimeError):
    def __init__(self, name, code):
        self.code = code
        if code == 2000:
            msg = f"{name}: the workspace installed for this stream is too small"
        elif code == 3000:
            msg = f"{name}: the call needs more than the static array's {STATIC_SCRATCH_BYTES} bytes"
        elif code == 3001:
            msg = f"{name}: the selected configuration is not a row-strip one"
        elif code == 3002:
            msg = f"{name}: device index beyond the static table"
        elif code >= 1000:
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
_GENTRY = {"s": "xgemv_s", "d": "xgemv_d", "c": "xgemv_c", "z": "xgemv_z", "w": "xgemv_w"}
_RENTRY = {"s": "xsyr2_s", "d": "xsyr2_d", "c": "xher2_c", "z": "xher2_z", "w": "xsyr2_w"}
_TENTRY = {"s": "xtrmv_s", "d": "xtrmv_d", "c": "xtrmv_c", "z": "xtrmv_z", "w": "xtrmv_w"}
_SHENTRY = {"s": "xsymv_shard_s", "d": "xsymv_shard_d", "c": "xhemv_shard_c",
            "z": "xhemv_shard_z", "w": "xsymv_shard_w"}
_CBENTRY = {"s": "xsymv_combine_s", "d": "xsymv_combine_d", "c": "xhemv_combine_c",
            "z": "xhemv_combine_z", "w": "xsymv_combine_w"}

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
            # torch carries its own HIP runtime: load it first, so that this
            # library's HIP dependency resolves to the same runtime and the
            # process holds one (two runtimes in one process do not share
            # the device: calls through the second fail with "no device")
            try:
                import torch  # noqa: F401
            except ImportError:
                pass
            lib = ctypes.CDLL(LIB_PATH)
            vp, ci, cc = ctypes.c_void_p, ctypes.c_int, ctypes.c_char
            for p, nm in _ENTRY.items():
                f = getattr(lib, nm)
                st = _SCALAR[p]
                f.restype = ci
                f.argtypes = [cc, ci, st, vp, ci, vp, ci, st, vp, ci, vp]
            for p, nm in _GENTRY.items():
                f = getattr(lib, nm)
                st = _SCALAR[p]
                f.restype = ci
                f.argtypes = [cc, ci, ci, st, vp, ci, vp, ci, st, vp, ci, vp]
            for p, nm in _RENTRY.items():
                f = getattr(lib, nm)
                f.restype = ci
                f.argtypes = [cc, ci, _SCALAR[p], vp, ci, vp, ci, vp, ci, vp]
            for p, nm in _TENTRY.items():
                f = getattr(lib, nm)
                f.restype = ci
                f.argtypes = [cc, cc, cc, ci, vp, ci, vp, ci, vp]
            for p, nm in _SHENTRY.items():
                f = getattr(lib, nm)
                f.restype = ci
                f.argtypes = [cc, ci, ci, ci, ci, vp, ci, vp, ci, vp, vp]
            for p, nm in _CBENTRY.items():
                f = getattr(lib, nm)
                f.restype = ci
                f.argtypes = [ci, ci, _SCALAR[p], vp, ci, _SCALAR[p], vp, ci, vp]
            lib.xsymv_shard_plan.restype = ci
            lib.xsymv_shard_plan.argtypes = [cc, ci, ci, ci, ci, ci, ci, ci, vp, ci, vp, vp, vp,
                                             ci]
            lib.xsymv_shard_columns.restype = ci
            lib.xsymv_shard_columns.argtypes = [ci, ci, ci, ci, vp]
            lib.xsymv_shard_workspace_bytes.restype = ctypes.c_size_t
            lib.xsymv_shard_workspace_bytes.argtypes = [ci, cc, ci, ci, ci, ci]
            lib.xtrmv_num_configs.restype = ci
            lib.xtrmv_num_configs.argtypes = [ci]
            lib.xtrmv_config_info.restype = ci
            lib.xtrmv_config_info.argtypes = [ci, ci] + [ctypes.POINTER(ci)] * 6
            lib.xtrmv_select_config.restype = ci
            lib.xtrmv_select_config.argtypes = [ci, ci]
            lib.xtrmv_current_config.restype = ci
            lib.xtrmv_current_config.argtypes = [ci, cc, cc, ci]
            lib.xtrmv_workspace_bytes.restype = ctypes.c_size_t
            lib.xtrmv_workspace_bytes.argtypes = [ci, cc, cc, ci]
            lib.xsymv_workspace_bytes.restype = ctypes.c_size_t
            lib.xsymv_workspace_bytes.argtypes = [ci, cc, ci]
            lib.xsymv_release.restype = ci
            lib.xsymv_release.argtypes = []
            lib.xsymv_set_workspace.restype = ci
            lib.xsymv_set_workspace.argtypes = [vp, ctypes.c_size_t, vp]
            lib.xsymv_num_configs.restype = ci
            lib.xsymv_num_configs.argtypes = [ci]
            ip = ctypes.POINTER(ci)
            fp = ctypes.POINTER(ctypes.c_float)
            lib.xsymv_config_info.restype = ci
            lib.xsymv_config_info.argtypes = [ci, ci, ip, ip, ip, ip, ip, ip, ip]
            lib.xsymv_select_config.restype = ci
            lib.xsymv_select_config.argtypes = [ci, cc, ci, ci, ci]
            lib.xsymv_current_config.restype = ci
            lib.xsymv_current_config.argtypes = [ci, cc, ci]
            lib.xsymv_current_config_lda.restype = ci
            lib.xsymv_current_config_lda.argtypes = [ci, cc, ci, ci]
            lib.xsymv_timing_enable.restype = ci
            lib.xsymv_timing_enable.argtypes = [ci]
            lib.xsymv_timing_read.restype = ci
            lib.xsymv_timing_read.argtypes = [fp, fp, ci]
            lib.xsymv_autotune.restype = ci
            lib.xsymv_autotune.argtypes = [ci, cc, ci, ci, ci, ci, vp, ip, fp, ci]
            lib.xsymv_autotune_lda.restype = ci
            lib.xsymv_autotune_lda.argtypes = [ci, cc, ci, ci, ci, ci, ci, vp, ip, fp, ci]
            for nm in ("xsymv_save_config", "xsymv_load_config"):
                getattr(lib, nm).restype = ci
                getattr(lib, nm).argtypes = [ctypes.c_char_p]
            lib.xsymv_s_noalloc.restype = ci
            lib.xsymv_s_noalloc.argtypes = [cc, ci, ctypes.c_float, vp, ci, vp, ci,
                                            ctypes.c_float, vp, ci, vp]
            lib.xsymv_clear_config.restype = ci
            lib.xsymv_clear_config.argtypes = []
            lib.xsymv_config_workgroups.restype = ci
            lib.xsymv_config_workgroups.argtypes = [ci, ci, cc]
            lib.xsymv_strip_plan.restype = ci
            lib.xsymv_strip_plan.argtypes = [cc, ci, ci, ci, ci, ip, ci, ip, ip, ci]
            lib.xsyr2_num_configs.restype = ci
            lib.xsyr2_num_configs.argtypes = [ci]
            lib.xsyr2_config_info.restype = ci
            lib.xsyr2_config_info.argtypes = [ci, ci, ip, ip, ip, ip, ip, ip]
            lib.xsyr2_select_config.restype = ci
            lib.xsyr2_select_config.argtypes = [ci, ci]
            lib.xsyr2_current_config.restype = ci
            lib.xsyr2_current_config.argtypes = [ci, cc, ci]
            lib.xgemv_num_configs.restype = ci
            lib.xgemv_num_configs.argtypes = [ci]
            lib.xgemv_config_info.restype = ci
            lib.xgemv_config_info.argtypes = [ci, ci, ip, ip, ip, ip, ip]
            lib.xgemv_select_config.restype = ci
            lib.xgemv_select_config.argtypes = [ci, ci]
            lib.xgemv_current_config.restype = ci
            lib.xgemv_current_config.argtypes = [ci, ctypes.c_char, ci, ci]
            lib.xgemv_workspace_bytes.restype = ctypes.c_size_t
            lib.xgemv_workspace_bytes.argtypes = [ci, cc, ci, ci]
            lib.xgemv_plan.restype = ci
            lib.xgemv_plan.argtypes = [ci, ci, ci, ci, ip, ci, ip, ci]
            lib.xsymv_read_bandwidth.restype = ci
            lib.xsymv_read_bandwidth.argtypes = [ctypes.c_size_t, ci, vp, fp, fp]
            lib.xsymv_copy_bandwidth.restype = ci
            lib.xsymv_copy_bandwidth.argtypes = [ctypes.c_size_t, ci, vp, fp, fp]
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


def xsymv_s_noalloc(uplo, n, alpha, A, lda, x, incx, beta, y, incy, stream=None):
    """SSYMV without device allocation: xsymv_s's product and bytes, its
    partial sums in the library's static array (shared by every call on the
    GPU: calls that overlap in time race)."""
    f = library().xsymv_s_noalloc
    u = uplo.encode()[:1] if isinstance(uplo, str) else uplo
    rc = f(u, n, _scalar("s", alpha), _addr(A), lda, _addr(x), incx, _scalar("s", beta),
           _addr(y), incy, _stream(stream))
    if rc != 0:
        raise XsymvError("xsymv_s_noalloc", rc)


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


def _gcall(prec, trans, m, n, alpha, A, lda, x, incx, beta, y, incy, stream):
    f = getattr(library(), _GENTRY[prec])
    t = trans.encode()[:1] if isinstance(trans, str) else trans
    rc = f(t, m, n, _scalar(prec, alpha), _addr(A), lda, _addr(x), incx,
           _scalar(prec, beta), _addr(y), incy, _stream(stream))
    if rc != 0:
        raise XsymvError(_GENTRY[prec], rc)


def xgemv_s(trans, m, n, alpha, A, lda, x, incx, beta, y, incy, stream=None):
    """SGEMV: y := alpha*op(A)*x + beta*y, float32, A m x n."""
    _gcall("s", trans, m, n, alpha, A, lda, x, incx, beta, y, incy, stream)


def xgemv_d(trans, m, n, alpha, A, lda, x, incx, beta, y, incy, stream=None):
    """DGEMV: float64."""
    _gcall("d", trans, m, n, alpha, A, lda, x, incx, beta, y, incy, stream)


def xgemv_c(trans, m, n, alpha, A, lda, x, incx, beta, y, incy, stream=None):
    """CGEMV: complex64 ('C' conjugates)."""
    _gcall("c", trans, m, n, alpha, A, lda, x, incx, beta, y, incy, stream)


def xgemv_z(trans, m, n, alpha, A, lda, x, incx, beta, y, incy, stream=None):
    """ZGEMV: complex128."""
    _gcall("z", trans, m, n, alpha, A, lda, x, incx, beta, y, incy, stream)


def xgemv_w(trans, m, n, alpha, A, lda, x, incx, beta, y, incy, stream=None):
    """WGEMV: double-double (hi, lo) pairs; alpha, beta are (hi, lo) tuples."""
    _gcall("w", trans, m, n, alpha, A, lda, x, incx, beta, y, incy, stream)


def _rcall(prec, uplo, n, alpha, x, incx, y, incy, A, lda, stream):
    f = getattr(library(), _RENTRY[prec])
    u = uplo.encode()[:1] if isinstance(uplo, str) else uplo
    rc = f(u, n, _scalar(prec, alpha), _addr(x), incx, _addr(y), incy, _addr(A), lda,
           _stream(stream))
    if rc != 0:
        raise XsymvError(_RENTRY[prec], rc)


def xsyr2_s(uplo, n, alpha, x, incx, y, incy, A, lda, stream=None):
    """SSYR2: A := alpha*x*y^T + alpha*y*x^T + A on the stored triangle, float32."""
    _rcall("s", uplo, n, alpha, x, incx, y, incy, A, lda, stream)


def xsyr2_d(uplo, n, alpha, x, incx, y, incy, A, lda, stream=None):
    """DSYR2: float64."""
    _rcall("d", uplo, n, alpha, x, incx, y, incy, A, lda, stream)


def xher2_c(uplo, n, alpha, x, incx, y, incy, A, lda, stream=None):
    """CHER2: A := alpha*x*y^H + conj(alpha)*y*x^H + A, complex64."""
    _rcall("c", uplo, n, alpha, x, incx, y, incy, A, lda, stream)


def xher2_z(uplo, n, alpha, x, incx, y, incy, A, lda, stream=None):
    """ZHER2: complex128."""
    _rcall("z", uplo, n, alpha, x, incx, y, incy, A, lda, stream)


def xsyr2_w(uplo, n, alpha, x, incx, y, incy, A, lda, stream=None):
    """WSYR2: double-double; alpha is a (hi, lo) tuple."""
    _rcall("w", uplo, n, alpha, x, incx, y, incy, A, lda, stream)


def _ch(v):
    return v.encode()[:1] if isinstance(v, str) else v


def _tcall(prec, uplo, trans, diag, n, A, lda, x, incx, stream):
    f = getattr(library(), _TENTRY[prec])
    rc = f(_ch(uplo), _ch(trans), _ch(diag), n, _addr(A), lda, _addr(x), incx, _stream(stream))
    if rc != 0:
        raise XsymvError(_TENTRY[prec], rc)


def xtrmv_s(uplo, trans, diag, n, A, lda, x, incx, stream=None):
    """STRMV: x := op(T)*x in place, T the stored triangle, float32."""
    _tcall("s", uplo, trans, diag, n, A, lda, x, incx, stream)


def xtrmv_d(uplo, trans, diag, n, A, lda, x, incx, stream=None):
    """DTRMV: float64."""
    _tcall("d", uplo, trans, diag, n, A, lda, x, incx, stream)


def xtrmv_c(uplo, trans, diag, n, A, lda, x, incx, stream=None):
    """CTRMV: complex64 ('C' conjugates)."""
    _tcall("c", uplo, trans, diag, n, A, lda, x, incx, stream)


def xtrmv_z(uplo, trans, diag, n, A, lda, x, incx, stream=None):
    """ZTRMV: complex128."""
    _tcall("z", uplo, trans, diag, n, A, lda, x, incx, stream)


def xtrmv_w(uplo, trans, diag, n, A, lda, x, incx, stream=None):
    """WTRMV: double-double (hi, lo) pairs."""
    _tcall("w", uplo, trans, diag, n, A, lda, x, incx, stream)


def _shcall(prec, uplo, n, panel, nshards, shard, Aloc, lda, x, incx, p, stream):
    f = getattr(library(), _SHENTRY[prec])
    rc = f(_ch(uplo), n, panel, nshards, shard, _addr(Aloc), lda, _addr(x), incx, _addr(p),
           _stream(stream))
    if rc != 0:
        raise XsymvError(_SHENTRY[prec], rc)


def xsymv_shard_s(uplo, n, panel, nshards, shard, Aloc, lda, x, incx, p, stream=None):
    """One shard's share p of S*x (float32): its own panels of columns, held
    as the local matrix Aloc, each stored element in both roles."""
    _shcall("s", uplo, n, panel, nshards, shard, Aloc, lda, x, incx, p, stream)


def xsymv_shard_d(uplo, n, panel, nshards, shard, Aloc, lda, x, incx, p, stream=None):
    """float64."""
    _shcall("d", uplo, n, panel, nshards, shard, Aloc, lda, x, incx, p, stream)


def xhemv_shard_c(uplo, n, panel, nshards, shard, Aloc, lda, x, incx, p, stream=None):
    """complex64, Hermitian."""
    _shcall("c", uplo, n, panel, nshards, shard, Aloc, lda, x, incx, p, stream)


def xhemv_shard_z(uplo, n, panel, nshards, shard, Aloc, lda, x, incx, p, stream=None):
    """complex128, Hermitian."""
    _shcall("z", uplo, n, panel, nshards, shard, Aloc, lda, x, incx, p, stream)


def xsymv_shard_w(uplo, n, panel, nshards, shard, Aloc, lda, x, incx, p, stream=None):
    """double-double."""
    _shcall("w", uplo, n, panel, nshards, shard, Aloc, lda, x, incx, p, stream)


def _cbcall(prec, n, nshards, alpha, P, ldp, beta, y, incy, stream):
    f = getattr(library(), _CBENTRY[prec])
    rc = f(n, nshards, _scalar(prec, alpha), _addr(P), ldp, _scalar(prec, beta), _addr(y), incy,
           _stream(stream))
    if rc != 0:
        raise XsymvError(_CBENTRY[prec], rc)


def xsymv_combine_s(n, nshards, alpha, P, ldp, beta, y, incy, stream=None):
    """y := beta*y + alpha*(P[0] + ... + P[nshards-1]) in rank order, float32."""
    _cbcall("s", n, nshards, alpha, P, ldp, beta, y, incy, stream)


def xsymv_combine_d(n, nshards, alpha, P, ldp, beta, y, incy, stream=None):
    """float64."""
    _cbcall("d", n, nshards, alpha, P, ldp, beta, y, incy, stream)


def xhemv_combine_c(n, nshards, alpha, P, ldp, beta, y, incy, stream=None):
    """complex64."""
    _cbcall("c", n, nshards, alpha, P, ldp, beta, y, incy, stream)


def xhemv_combine_z(n, nshards, alpha, P, ldp, beta, y, incy, stream=None):
    """complex128."""
    _cbcall("z", n, nshards, alpha, P, ldp, beta, y, incy, stream)


def xsymv_combine_w(n, nshards, alpha, P, ldp, beta, y, incy, stream=None):
    """double-double; alpha, beta are (hi, lo) tuples."""
    _cbcall("w", n, nshards, alpha, P, ldp, beta, y, incy, stream)


def shard_columns(n: int, panel: int, nshards: int, shard: int):
    """Global columns of a shard (ascending), as a list."""
    lib = library()
    k = lib.xsymv_shard_columns(n, panel, nshards, shard, None)
    if k < 0:
        raise ValueError("bad shard arguments")
    buf = (ctypes.c_int * max(k, 1))()
    lib.xsymv_shard_columns(n, panel, nshards, shard, buf)
    return list(buf[:k])


def shard_plan(uplo: str, n: int, R: int, G: int, split: int, panel: int, nshards: int,
               shard: int):
    """One shard's work split (host computation): (blocks [k x 4],
    strip_base [NS+1], seg_base [NS+1], col0 [NS])."""
    import numpy as np
    ns = (n + R - 1) // R
    blocks = np.zeros((G, 4), dtype=np.int32)
    sb = np.zeros(ns + 1, dtype=np.int32)
    segb = np.zeros(ns + 1, dtype=np.int32)
    c0 = np.zeros(ns + 1, dtype=np.int32)
    k = library().xsymv_shard_plan(_ch(uplo), n, R, G, split, panel, nshards, shard,
                                   blocks.ctypes.data, G, sb.ctypes.data, segb.ctypes.data,
                                   c0.ctypes.data, ns + 1)
    if k < 0:
        raise ValueError(f"xsymv_shard_plan failed ({k})")
    return blocks[:k], sb, segb, c0[:ns]


def shard_workspace_bytes(prec: str, uplo: str, n: int, panel: int, nshards: int,
                          shard: int) -> int:
    v = library().xsymv_shard_workspace_bytes(PREC_CODE[prec], _ch(uplo), n, panel, nshards,
                                              shard)
    if v == ctypes.c_size_t(-1).value:
        raise XsymvError("xsymv_shard_workspace_bytes", 1000)
    return v


def trmv_num_configs(prec: str) -> int:
    return library().xtrmv_num_configs(PREC_CODE[prec])


def trmv_config_info(prec: str, idx: int) -> dict:
    vals = [ctypes.c_int() for _ in range(6)]
    if library().xtrmv_config_info(PREC_CODE[prec], idx, *[ctypes.byref(v) for v in vals]) != 0:
        raise IndexError(idx)
    w, sw, g, nt, sp, r = (v.value for v in vals)
    return {"waves": w, "stripes_per_wave": sw, "cols_per_group": g, "nontemporal": nt,
            "split": sp, "rows_per_strip": r}


def trmv_select_config(prec: str, idx: int) -> None:
    if library().xtrmv_select_config(PREC_CODE[prec], idx) != 0:
        raise ValueError("bad trmv configuration selection")


def trmv_current_config(prec: str, uplo: str, trans: str, n: int) -> int:
    """The configuration a call (prec, uplo, trans, n) would use now."""
    v = library().xtrmv_current_config(PREC_CODE[prec], _ch(uplo), _ch(trans), n)
    if v < 0:
        raise ValueError("bad trmv configuration query")
    return v


def trmv_workspace_bytes(prec: str, uplo: str, trans: str, n: int) -> int:
    """Device workspace bytes of one call with the selected configuration
    (needs the device: the split depends on resident workgroups)."""
    v = library().xtrmv_workspace_bytes(PREC_CODE[prec], _ch(uplo), _ch(trans), n)
    if v == ctypes.c_size_t(-1).value:
        raise XsymvError("xtrmv_workspace_bytes", 1000)
    return v


def syr2_num_configs(prec: str) -> int:
    return library().xsyr2_num_configs(PREC_CODE[prec])


def syr2_config_info(prec: str, idx: int) -> dict:
    vals = [ctypes.c_int() for _ in range(6)]
    if library().xsyr2_config_info(PREC_CODE[prec], idx, *[ctypes.byref(v) for v in vals]) != 0:
        raise IndexError(idx)
    w, sw, g, nt, sp, r = (v.value for v in vals)
    return {"waves": w, "stripes_per_wave": sw, "cols_per_group": g, "nontemporal": nt,
            "split": sp, "rows_per_strip": r}


def syr2_select_config(prec: str, idx: int) -> None:
    """Force configuration idx for every rank-2 update of `prec`; -1 restores
    the built-in choice per triangle and size."""
    if library().xsyr2_select_config(PREC_CODE[prec], idx) != 0:
        raise ValueError("bad syr2 configuration selection")


def syr2_current_config(prec: str, uplo: str, n: int) -> int:
    """The configuration a rank-2 update (prec, uplo, n) runs."""
    v = library().xsyr2_current_config(PREC_CODE[prec], _ch(uplo), n)
    if v < 0:
        raise ValueError("bad syr2 configuration query")
    return v


def gemv_num_configs(prec: str) -> int:
    return library().xgemv_num_configs(PREC_CODE[prec])


def gemv_config_info(prec: str, idx: int) -> dict:
    vals = [ctypes.c_int() for _ in range(5)]
    if library().xgemv_config_info(PREC_CODE[prec], idx, *[ctypes.byref(v) for v in vals]) != 0:
        raise IndexError(idx)
    w, sw, g, nt, r = (v.value for v in vals)
    return {"waves": w, "stripes_per_wave": sw, "cols_per_group": g, "nontemporal": nt,
            "rows_per_strip": r}


def gemv_select_config(prec: str, idx: int) -> None:
    """Force configuration idx for every xGEMV call of `prec`; -1 restores
    the built-in choice per transposition and size."""
    if library().xgemv_select_config(PREC_CODE[prec], idx) != 0:
        raise ValueError("bad gemv configuration selection")


def gemv_current_config(prec: str, trans: str, m: int, n: int) -> int:
    """The configuration an xGEMV call (prec, trans, m, n) runs."""
    return library().xgemv_current_config(PREC_CODE[prec], trans.encode()[:1], m, n)


def gemv_workspace_bytes(prec: str, trans: str, m: int, n: int) -> int:
    return library().xgemv_workspace_bytes(PREC_CODE[prec], trans.encode()[:1], m, n)


def gemv_plan(m: int, n: int, R: int, G: int):
    """The xGEMV work split (host computation): (blocks [G x 4], seg_base [NS+1])."""
    import numpy as np
    ns = (m + R - 1) // R
    blocks = np.zeros((G, 4), dtype=np.int32)
    segb = np.zeros(ns + 1, dtype=np.int32)
    ip = ctypes.POINTER(ctypes.c_int)
    k = library().xgemv_plan(m, n, R, G, blocks.ctypes.data_as(ip), G,
                             segb.ctypes.data_as(ip), ns + 1)
    if k < 0:
        raise ValueError(f"xgemv_plan failed ({k})")
    return blocks[:k], segb


def workspace_bytes(prec: str, uplo: str, n: int) -> int:
    return library().xsymv_workspace_bytes(PREC_CODE[prec], uplo.encode()[:1], n)


def num_configs(prec: str) -> int:
    return library().xsymv_num_configs(PREC_CODE[prec])


def config_info(prec: str, idx: int) -> dict:
    vals = [ctypes.c_int() for _ in range(7)]
    rc = library().xsymv_config_info(PREC_CODE[prec], idx, *[ctypes.byref(v) for v in vals])
    if rc != 0:
        raise IndexError(idx)
    w, cw, s, h, nt, xl, cr = (v.value for v in vals)
    return {"waves": w, "cols_per_wave": cw, "stripes": s, "rows_per_stripe": h,
            "nontemporal": nt, "x_in_lds": xl, "column_runs": cr, "panel": w * cw,
            "tile_rows": s * h}


def select_config(prec: str, uplo: str, n_lo: int, n_hi: int, idx: int) -> None:
    rc = library().xsymv_select_config(PREC_CODE[prec], uplo.encode()[:1], n_lo, n_hi, idx)
    if rc != 0:
        raise ValueError("bad configuration selection")


def current_config(prec: str, uplo: str, n: int, lda: int | None = None) -> int:
    """The configuration a call would use now (``lda`` default: a leading
    dimension whose columns are whole 64-byte lines)."""
    if lda is None:
        return library().xsymv_current_config(PREC_CODE[prec], uplo.encode()[:1], n)
    return library().xsymv_current_config_lda(PREC_CODE[prec], uplo.encode()[:1], n, lda)


def autotune(prec: str, uplo: str, n: int, n_lo: int | None = None, n_hi: int | None = None,
             reps: int = 10, stream=None, lda: int | None = None):
    """Time every compiled configuration for (prec, uplo, n) on the device
    (on a matrix of leading dimension ``lda``, default n), install the
    fastest for n in [n_lo, n_hi] (default: n only) and return (best index,
    list of median milliseconds per configuration)."""
    k = num_configs(prec)
    ms = (ctypes.c_float * k)()
    best = ctypes.c_int(-1)
    n_lo = n if n_lo is None else n_lo
    n_hi = n if n_hi is None else n_hi
    lda = n if lda is None else lda
    rc = library().xsymv_autotune_lda(PREC_CODE[prec], uplo.encode()[:1], n, lda, n_lo, n_hi,
                                      reps, _stream(stream), ctypes.byref(best), ms, k)
    if rc != 0:
        raise XsymvError("xsymv_autotune_lda", rc)
    return best.value, list(ms)


def save_config(path: str) -> None:
    if library().xsymv_save_config(os.fsencode(path)) != 0:
        raise OSError(f"cannot write {path}")


def load_config(path: str) -> int:
    """Install the rules of a JSON file; returns how many were installed."""
    k = library().xsymv_load_config(os.fsencode(path))
    if k == -1:
        raise OSError(f"cannot read {path}")
    if k == -2:
        raise ValueError(f"malformed rule file {path}")
    return k


def clear_config() -> None:
    library().xsymv_clear_config()


def timing_enable(mode) -> None:
    """Timing mode: False/0 off, True/1 main kernel and merge per call, 2 each
    call whole (no event bound between its kernels)."""
    m = int(mode)
    if library().xsymv_timing_enable(m) != 0:
        raise ValueError(f"timing mode {mode!r}: 0, 1 or 2")


def timing_read(max_calls: int = 4096):
    """List of (main_ms, merge_ms) for the calls recorded since timing was
    enabled or last read: mode 1 the main kernel and, from its end, the
    merge; mode 2 (call span, 0)."""
    a = (ctypes.c_float * max_calls)()
    b = (ctypes.c_float * max_calls)()
    k = library().xsymv_timing_read(a, b, max_calls)
    if k >= 1000:
        raise XsymvError("xsymv_timing_read", k)
    return [(a[i], b[i]) for i in range(k)]


def config_workgroups(prec: str, idx: int, uplo: str = "L") -> int:
    """Workgroups a row-strip configuration is launched with (0 otherwise)."""
    return library().xsymv_config_workgroups(PREC_CODE[prec], idx, uplo.encode()[:1])


def strip_plan(uplo: str, n: int, R: int, G: int, split: int = 0):
    """The row-strip work split (host computation) under cost model `split`
    (0: strip height per column, doubled in the triangle; 1: stored rows plus
    strip height; 2: strip height alone): (blocks [G x 4]: first, end, first slot, first strip),
    strip_base [NS+1], seg_base [NS+1]."""
    import numpy as np
    ns = (n + R - 1) // R
    blocks = np.zeros((G, 4), dtype=np.int32)
    sb = np.zeros(ns + 1, dtype=np.int32)
    segb = np.zeros(ns + 1, dtype=np.int32)
    ip = ctypes.POINTER(ctypes.c_int)
    k = library().xsymv_strip_plan(uplo.encode()[:1], n, R, G, split, blocks.ctypes.data_as(ip), G,
                                    sb.ctypes.data_as(ip), segb.ctypes.data_as(ip), ns + 1)
    if k < 0:
        raise ValueError(f"xsymv_strip_plan failed ({k})")
    return blocks[:k], sb, segb


def set_workspace(buf, nbytes: int | None = None, stream=None) -> None:
    """Install a caller-owned device buffer (a torch tensor or an address) as
    the workspace of `stream`; ``None`` removes it.  ``nbytes`` defaults to
    the tensor's size in bytes."""
    if buf is None:
        ptr, nbytes = None, 0
    else:
        ptr = _addr(buf)
        if nbytes is None:
            nbytes = buf.numel() * buf.element_size()
    rc = library().xsymv_set_workspace(ptr, nbytes, _stream(stream))
    if rc != 0:
        raise XsymvError("xsymv_set_workspace", rc)


def read_bandwidth(nbytes: int = 4 << 30, reps: int = 10, stream=None):
    """(median, best) GB/s of a plain streaming read of ``nbytes`` on the device."""
    med = ctypes.c_float()
    best = ctypes.c_float()
    rc = library().xsymv_read_bandwidth(nbytes, reps, _stream(stream), ctypes.byref(med),
                                        ctypes.byref(best))
    if rc != 0:
        raise XsymvError("xsymv_read_bandwidth", rc)
    return med.value, best.value


def copy_bandwidth(nbytes: int = 2 << 30, reps: int = 10, stream=None):
    """(median, best) GB/s, bytes read plus bytes written, of a plain copy of
    ``nbytes`` on the device."""
    med = ctypes.c_float()
    best = ctypes.c_float()
    rc = library().xsymv_copy_bandwidth(nbytes, reps, _stream(stream), ctypes.byref(med),
                                        ctypes.byref(best))
    if rc != 0:
        raise XsymvError("xsymv_copy_bandwidth", rc)
    return med.value, best.value


def release() -> None:
    rc = library().xsymv_release()
    if rc != 0:
        raise XsymvError("xsymv_release", rc)


def version() -> str:
    return library().xsymv_version().decode()
