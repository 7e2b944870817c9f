"""Checkers shared by the tests: explicit symmetrisation, exact products,
the componentwise error bound, comparisons.

They are written from the definition of the product (the CUDA-xSYMV report,
§1 eq.(1)) and share nothing with either the oracle or the GPU library.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

# unit roundoff per element type (2^-24, 2^-53; double-double 2^-104)
EPS = {"s": 2.0 ** -24, "c": 2.0 ** -24, "d": 2.0 ** -53, "z": 2.0 ** -53,
       "w": 2.0 ** -104}


def is_upper(uplo: str) -> bool:
    return uplo in ("U", "u")


def stored(uplo: str, i: int, j: int) -> bool:
    return i <= j if is_upper(uplo) else i >= j


def vec_index(n: int, inc: int) -> np.ndarray:
    """Storage positions of logical elements 0..n-1 of a strided vector."""
    start = 0 if inc > 0 else (1 - n) * inc
    return start + np.arange(n, dtype=np.int64) * inc


def dense_matrix(p, dtype=None) -> np.ndarray:
    """Full n x n matrix implied by the stored triangle (conjugate mirror and
    real diagonal for Hermitian types), as complex128/float64 (double-double:
    hi + lo rounded to float64)."""
    n, lda = p.n, p.lda
    if p.prec == "w":
        A = p.A[:, 0].astype(np.float64) + p.A[:, 1]
    else:
        A = p.A
    M = A[: lda * n].reshape(n, lda).T[:n, :n]  # column-major -> [i, j]
    dt = dtype or (np.complex128 if p.prec in ("c", "z") else np.float64)
    M = M.astype(dt)
    low = np.tril(np.ones((n, n), dtype=bool), -1)
    if is_upper(p.uplo):
        S = np.where(low, np.conj(M.T), M)
    else:
        S = np.where(low.T, np.conj(M.T), M)
    S = np.array(S)
    d = np.arange(n)
    if p.prec in ("c", "z"):
        S[d, d] = M[d, d].real
    return S


def _frac(v) -> Fraction:
    return Fraction(float(v))


def exact_elements(p):
    """Stored elements as exact values: Fraction (real, double-double) or a
    pair of Fractions (complex)."""
    n, lda = p.n, p.lda

    def get(i, j):
        k = i + j * lda
        if p.prec == "w":
            return Fraction(float(p.A[k, 0])) + Fraction(float(p.A[k, 1]))
        if p.prec in ("c", "z"):
            return (_frac(p.A[k].real), _frac(p.A[k].imag))
        return _frac(p.A[k])

    return get


def exact_vector(p, v, inc):
    idx = vec_index(p.n, inc)
    if p.prec == "w":
        return [Fraction(float(v[k, 0])) + Fraction(float(v[k, 1])) for k in idx]
    if p.prec in ("c", "z"):
        return [(_frac(v[k].real), _frac(v[k].imag)) for k in idx]
    return [_frac(v[k]) for k in idx]


def exact_scalar(prec, s):
    if prec == "w":
        return Fraction(float(s[0])) + Fraction(float(s[1]))
    if prec in ("c", "z"):
        c = complex(s)
        return (Fraction(c.real), Fraction(c.imag))
    return Fraction(float(s))


def _cmul(a, b):
    return (a[0] * b[0] - a[1] * b[1], a[0] * b[1] + a[1] * b[0])


def _cadd(a, b):
    return (a[0] + b[0], a[1] + b[1])


def exact_result(p):
    """Exact alpha*S*x + beta*y (y ignored when beta == 0), as a list of
    Fractions or (re, im) Fraction pairs, in logical order."""
    n = p.n
    get = exact_elements(p)
    cplx = p.prec in ("c", "z")
    x = exact_vector(p, p.x, p.incx)
    al = exact_scalar(p.prec, p.alpha)
    be = exact_scalar(p.prec, p.beta)
    beta_zero = be == (0, 0) if cplx else be == 0
    y = None if beta_zero else exact_vector(p, p.y, p.incy)
    out = []
    zero = (Fraction(0), Fraction(0)) if cplx else Fraction(0)
    for i in range(n):
        s = zero
        for j in range(n):
            if i == j:
                a = get(i, i)
                if cplx:
                    a = (a[0], Fraction(0))
            elif stored(p.uplo, i, j):
                a = get(i, j)
            else:
                a = get(j, i)
                if cplx:
                    a = (a[0], -a[1])
            s = _cadd(s, _cmul(a, x[j])) if cplx else s + a * x[j]
        if cplx:
            r = _cmul(al, s)
            if not beta_zero:
                r = _cadd(r, _cmul(be, y[i]))
        else:
            r = al * s
            if not beta_zero:
                r = r + be * y[i]
        out.append(r)
    return out


def abs_bound_terms(p):
    """(|alpha|*(|S||x|)_i + |beta|*|y_i|) in float64, logical order."""
    S = np.abs(dense_matrix(p))
    xi = vec_index(p.n, p.incx)
    yi = vec_index(p.n, p.incy)
    if p.prec == "w":
        x = np.abs(p.x[xi, 0] + p.x[xi, 1])
        y = np.abs(p.y[yi, 0] + p.y[yi, 1])
        al = abs(p.alpha[0] + p.alpha[1])
        be = abs(p.beta[0] + p.beta[1])
    else:
        x = np.abs(p.x[xi]).astype(np.float64)
        y = np.abs(p.y[yi]).astype(np.float64)
        al = abs(complex(p.alpha))
        be = abs(complex(p.beta))
    t = al * (S @ x)
    if be != 0:
        t = t + be * np.where(np.isfinite(y), y, 0.0)
    return t


def _scalar_magnitudes(p):
    if p.prec == "w":
        return abs(p.alpha[0] + p.alpha[1]), abs(p.beta[0] + p.beta[1])
    return abs(complex(p.alpha)), abs(complex(p.beta))


def abs_bound_blocked(p, block: int = 512):
    """(|alpha|*(|S||x|)_i + |beta|*|y_i|) for every logical row, read from
    the stored triangle one block of columns at a time (no n x n array), so
    that it serves the largest orders: a stored element A(r, c) adds
    |A(r, c)||x_c| to row r and, off the diagonal, |A(r, c)||x_r| to row c
    (|S| is symmetric).  A Hermitian diagonal counts its real word only."""
    n, lda = p.n, p.lda
    ax = _magnitude(p, p.x[vec_index(n, p.incx)])
    ay = _magnitude(p, p.y[vec_index(n, p.incy)])
    al, be = _scalar_magnitudes(p)
    up = is_upper(p.uplo)
    t = np.zeros(n)
    for c0 in range(0, n, block):
        c1 = min(n, c0 + block)
        # rows holding stored elements of these columns: U [0, c1), L [c0, n)
        r0, r1 = (0, c1) if up else (c0, n)
        blk = p.A[c0 * lda:c1 * lda]
        blk = blk.reshape(c1 - c0, lda, 2)[:, r0:r1] if p.prec == "w" else \
            blk.reshape(c1 - c0, lda)[:, r0:r1]
        if p.prec == "w":
            M = np.abs(blk[..., 0] + blk[..., 1])    # M[c - c0, r - r0] = |A(r, c)|
        else:
            M = np.abs(blk.astype(np.complex128 if p.prec in ("c", "z") else np.float64))
        # the diagonal square [c0, c1): keep the stored side only
        k = np.arange(c1 - c0)
        sq = M[:, c0 - r0:c1 - r0]
        keep = (k[None, :] <= k[:, None]) if up else (k[None, :] >= k[:, None])
        sq[~keep] = 0.0
        if p.prec in ("c", "z"):
            sq[k, k] = np.abs(blk[k, c0 - r0 + k].real.astype(np.float64))
        t[r0:r1] += ax[c0:c1] @ M                     # row role, diagonal included
        sq[k, k] = 0.0
        t[c0:c1] += M @ ax[r0:r1]                     # mirrored role
    t = al * t
    if be != 0:
        t = t + be * np.where(np.isfinite(ay), ay, 0.0)
    return t


def tolerance(p, rows=None):
    """Componentwise bound 4*n*eps*(|alpha|*(|S||x|)_i + |beta|*|y_i|), for all
    rows (read block by block from the stored triangle) or for the logical
    rows ``rows`` only."""
    if rows is None:
        return 4.0 * max(p.n, 1) * EPS[p.prec] * abs_bound_blocked(p)
    return 4.0 * max(p.n, 1) * EPS[p.prec] * abs_bound_rows(p, rows)


def _magnitude(p, v):
    if p.prec == "w":
        return np.abs(v[..., 0] + v[..., 1])
    return np.abs(v).astype(np.float64)


def abs_bound_rows(p, rows):
    """(|alpha|*(|S||x|)_i + |beta|*|y_i|) for logical rows ``rows``, read
    straight from the stored triangle (unit increments only)."""
    assert p.incx == 1 and p.incy == 1
    n, lda = p.n, p.lda
    ax = _magnitude(p, p.x)
    ay = _magnitude(p, p.y)
    if p.prec == "w":
        al = abs(p.alpha[0] + p.alpha[1])
        be = abs(p.beta[0] + p.beta[1])
    else:
        al = abs(complex(p.alpha))
        be = abs(complex(p.beta))
    out = np.empty(len(rows))
    j = np.arange(n, dtype=np.int64)
    for k, i in enumerate(rows):
        st = (j >= i) if is_upper(p.uplo) else (j <= i)
        idx = np.where(st, i + j * lda, j + i * lda)
        a = _magnitude(p, p.A[idx])
        if p.prec in ("c", "z"):
            a[i] = abs(float(p.A[i + i * lda].real))
        t = al * float(a @ ax)
        if be != 0 and np.isfinite(ay[i]):
            t += be * ay[i]
        out[k] = t
    return out


def exact_errors(p, y_out, exact=None):
    """|y_out - exact| per logical element, as float64 (exact subtraction in
    rationals, then rounded)."""
    ex = exact_result(p) if exact is None else exact
    idx = vec_index(p.n, p.incy)
    errs = np.empty(p.n)
    for k, i in enumerate(idx):
        e = ex[k]
        if p.prec == "w":
            v = Fraction(float(y_out[i, 0])) + Fraction(float(y_out[i, 1]))
            errs[k] = abs(float(v - e))
        elif p.prec in ("c", "z"):
            re = _frac(y_out[i].real) - e[0]
            im = _frac(y_out[i].imag) - e[1]
            errs[k] = abs(complex(float(re), float(im)))
        else:
            errs[k] = abs(float(_frac(y_out[i]) - e))
    return errs


def diff(prec, a, b):
    """|a - b| elementwise in float64; double-double as (hi-hi) + (lo-lo)."""
    if prec == "w":
        return np.abs((a[..., 0] - b[..., 0]) + (a[..., 1] - b[..., 1]))
    return np.abs(a.astype(np.complex128) - b.astype(np.complex128)) \
        if prec in ("c", "z") else np.abs(a.astype(np.float64) - b.astype(np.float64))


def integer_expected(p):
    """Exact result for integer-valued problems via int64 dense products, in
    the element type (every value involved is exactly representable)."""
    n = p.n
    M = dense_matrix(p)
    xi = vec_index(n, p.incx)
    yi = vec_index(n, p.incy)
    if p.prec in ("c", "z"):
        Sr = np.rint(M.real).astype(np.int64)
        Si = np.rint(M.imag).astype(np.int64)
        xr = np.rint(p.x[xi].real).astype(np.int64)
        xim = np.rint(p.x[xi].imag).astype(np.int64)
        sr = Sr @ xr - Si @ xim
        si = Sr @ xim + Si @ xr
        s = sr.astype(np.complex128) + 1j * si.astype(np.complex128)
        al = complex(p.alpha)
        be = complex(p.beta)
        y = p.y[yi].astype(np.complex128)
        out = al * s + (be * y if be != 0 else 0)
        return out.astype(p.y.dtype)
    S = np.rint(M).astype(np.int64)
    if p.prec == "w":
        x = np.rint(p.x[xi, 0]).astype(np.int64)
        y = p.y[yi, 0]
        al, be = p.alpha[0], p.beta[0]
    else:
        x = np.rint(p.x[xi]).astype(np.int64)
        y = p.y[yi].astype(np.float64)
        al, be = float(p.alpha), float(p.beta)
    s = (S @ x).astype(np.float64)
    out = al * s + (be * y if be != 0 else 0.0)
    if p.prec == "w":
        r = np.zeros((n, 2))
        r[:, 0] = out
        return r
    return out.astype(p.y.dtype)


def np_mul(a, b):
    """Elementwise product in the element type with one rounding per real
    operation (complex: textbook formula, each real product and sum rounded
    separately), independent of how numpy implements complex multiply."""
    if np.iscomplexobj(a) or np.iscomplexobj(b):
        dt = np.result_type(a, b)
        rt = np.float32 if dt == np.complex64 else np.float64
        a = np.asarray(a, dtype=dt)
        b = np.asarray(b, dtype=dt)
        ar, ai = a.real.astype(rt), a.imag.astype(rt)
        br, bi = b.real.astype(rt), b.imag.astype(rt)
        re = np.subtract(np.multiply(ar, br), np.multiply(ai, bi))
        im = np.add(np.multiply(ar, bi), np.multiply(ai, br))
        out = np.empty(np.broadcast(re, im).shape, dtype=dt)
        out.real = re
        out.imag = im
        return out
    return np.multiply(a, b)


# ------------------------------------------------------------------ xGEMV

def gemv_vec_index(length: int, inc: int) -> np.ndarray:
    return vec_index(length, inc)


def gemv_op_dense(p) -> np.ndarray:
    """op(A) as a dense (leny x lenx) float64/complex128 array (double-double:
    hi + lo rounded to float64)."""
    A = p.A[:, 0].astype(np.float64) + p.A[:, 1] if p.prec == "w" else p.A
    M = A[: p.lda * p.n].reshape(p.n, p.lda).T[: p.m, :]  # [i, j], m x n
    dt = np.complex128 if p.prec in ("c", "z") else np.float64
    M = M.astype(dt)
    if p.trans in ("N", "n"):
        return M
    return np.conj(M.T) if p.trans in ("C", "c") else M.T.copy()


def _gemv_exact_vec(p, v, length, inc):
    idx = vec_index(length, inc)
    if p.prec == "w":
        return [Fraction(float(v[k, 0])) + Fraction(float(v[k, 1])) for k in idx]
    if p.prec in ("c", "z"):
        return [(_frac(v[k].real), _frac(v[k].imag)) for k in idx]
    return [_frac(v[k]) for k in idx]


def gemv_exact(p):
    """Exact alpha*op(A)*x + beta*y in logical order (y ignored if beta == 0)."""
    cplx = p.prec in ("c", "z")
    tr = p.trans not in ("N", "n")
    conj = p.trans in ("C", "c")

    def get(i, j):
        k = i + j * p.lda
        if p.prec == "w":
            return Fraction(float(p.A[k, 0])) + Fraction(float(p.A[k, 1]))
        if cplx:
            return (_frac(p.A[k].real), _frac(p.A[k].imag))
        return _frac(p.A[k])

    x = _gemv_exact_vec(p, p.x, p.lenx, p.incx)
    al = exact_scalar(p.prec, p.alpha)
    be = exact_scalar(p.prec, p.beta)
    beta_zero = be == (0, 0) if cplx else be == 0
    y = None if beta_zero else _gemv_exact_vec(p, p.y, p.leny, p.incy)
    zero = (Fraction(0), Fraction(0)) if cplx else Fraction(0)
    out = []
    for o in range(p.leny):
        s = zero
        for k in range(p.lenx):
            a = get(k, o) if tr else get(o, k)
            if cplx:
                if conj:
                    a = (a[0], -a[1])
                s = _cadd(s, _cmul(a, x[k]))
            else:
                s = s + a * x[k]
        if cplx:
            r = _cmul(al, s)
            if not beta_zero:
                r = _cadd(r, _cmul(be, y[o]))
        else:
            r = al * s
            if not beta_zero:
                r = r + be * y[o]
        out.append(r)
    return out


def gemv_exact_errors(p, y_out, exact=None):
    ex = gemv_exact(p) if exact is None else exact
    idx = vec_index(p.leny, p.incy)
    errs = np.empty(p.leny)
    for k, i in enumerate(idx):
        e = ex[k]
        if p.prec == "w":
            v = Fraction(float(y_out[i, 0])) + Fraction(float(y_out[i, 1]))
            errs[k] = abs(float(v - e))
        elif p.prec in ("c", "z"):
            errs[k] = abs(complex(float(_frac(y_out[i].real) - e[0]),
                                  float(_frac(y_out[i].imag) - e[1])))
        else:
            errs[k] = abs(float(_frac(y_out[i]) - e))
    return errs


def gemv_tolerance(p, rows=None):
    """4*k*eps*(|alpha|*(|op(A)||x|)_i + |beta|*|y_i|), k = the inner length,
    for all outputs (logical order) or for the outputs ``rows`` only (unit
    increments, read column by column without forming op(A))."""
    k = max(p.lenx, 1)
    if p.prec == "w":
        al = abs(p.alpha[0] + p.alpha[1])
        be = abs(p.beta[0] + p.beta[1])
    else:
        al = abs(complex(p.alpha))
        be = abs(complex(p.beta))
    if rows is None:
        x = _magnitude(p, p.x[vec_index(p.lenx, p.incx)])
        y = _magnitude(p, p.y[vec_index(p.leny, p.incy)])
        t = al * (np.abs(gemv_op_dense(p)) @ x)
    else:
        assert p.incx == 1 and p.incy == 1
        rows = np.asarray(rows, dtype=np.int64)
        x = _magnitude(p, p.x)
        y = _magnitude(p, p.y)[rows]
        t = np.empty(len(rows))
        kk = np.arange(p.lenx, dtype=np.int64)
        for r, o in enumerate(rows):
            idx = (kk + o * p.lda) if p.trans not in ("N", "n") else (o + kk * p.lda)
            t[r] = al * float(_magnitude(p, p.A[idx]) @ x)
    if be != 0:
        t = t + be * np.where(np.isfinite(y), y, 0.0)
    return 4.0 * k * EPS[p.prec] * t


def gemv_integer_expected(p):
    """Exact result of an integer-valued GemvProblem via int64 products, in
    the element type."""
    M = gemv_op_dense(p)
    xi = vec_index(p.lenx, p.incx)
    yi = vec_index(p.leny, p.incy)
    if p.prec in ("c", "z"):
        Mr = np.rint(M.real).astype(np.int64)
        Mi = np.rint(M.imag).astype(np.int64)
        xr = np.rint(p.x[xi].real).astype(np.int64)
        xim = np.rint(p.x[xi].imag).astype(np.int64)
        s = (Mr @ xr - Mi @ xim).astype(np.complex128) + 1j * (Mr @ xim + Mi @ xr)
        al, be = complex(p.alpha), complex(p.beta)
        out = al * s + (be * p.y[yi].astype(np.complex128) if be != 0 else 0)
        return out.astype(p.y.dtype)
    Mi = np.rint(M).astype(np.int64)
    if p.prec == "w":
        x = np.rint(p.x[xi, 0]).astype(np.int64)
        y = p.y[yi, 0]
        al, be = p.alpha[0], p.beta[0]
    else:
        x = np.rint(p.x[xi]).astype(np.int64)
        y = p.y[yi].astype(np.float64)
        al, be = float(p.alpha), float(p.beta)
    out = al * (Mi @ x).astype(np.float64) + (be * y if be != 0 else 0.0)
    if p.prec == "w":
        r = np.zeros((p.leny, 2))
        r[:, 0] = out
        return r
    return out.astype(p.y.dtype)


# ------------------------------------------------------------------ xTRMV

def _trmv_unit(p) -> bool:
    return p.diag in ("U", "u")


def trmv_op_dense(p) -> np.ndarray:
    """op(T) as a dense n x n float64/complex128 array: T the stored triangle
    (zeros elsewhere, ones on the diagonal for a unit triangle; double-double
    hi + lo rounded to float64)."""
    n = p.n
    A = p.A[:, 0].astype(np.float64) + p.A[:, 1] if p.prec == "w" else p.A
    dt = np.complex128 if p.prec in ("c", "z") else np.float64
    M = A[: p.lda * n].reshape(n, p.lda).T[:n, :n].astype(dt)  # [i, j]
    keep = np.triu(np.ones((n, n), dtype=bool)) if is_upper(p.uplo) else \
        np.tril(np.ones((n, n), dtype=bool))
    T = np.where(keep, M, 0)
    if _trmv_unit(p):
        T[np.arange(n), np.arange(n)] = 1
    if p.trans in ("N", "n"):
        return T
    return np.conj(T.T) if p.trans in ("C", "c") else T.T.copy()


def trmv_exact(p):
    """Exact op(T)*x in logical order (Fractions or (re, im) Fraction pairs)."""
    cplx = p.prec in ("c", "z")
    tr = p.trans not in ("N", "n")
    conj = p.trans in ("C", "c")
    get = exact_elements(p)
    x = exact_vector(p, p.x, p.incx)
    zero = (Fraction(0), Fraction(0)) if cplx else Fraction(0)
    out = []
    for o in range(p.n):
        s = zero
        for k in range(p.n):
            r, c = (k, o) if tr else (o, k)
            if not stored(p.uplo, r, c):
                continue
            if r == c and _trmv_unit(p):
                s = _cadd(s, x[k]) if cplx else s + x[k]
                continue
            a = get(r, c)
            if cplx:
                if conj:
                    a = (a[0], -a[1])
                s = _cadd(s, _cmul(a, x[k]))
            else:
                s = s + a * x[k]
        out.append(s)
    return out


def trmv_exact_errors(p, x_out, exact=None):
    ex = trmv_exact(p) if exact is None else exact
    idx = vec_index(p.n, p.incx)
    errs = np.empty(p.n)
    for k, i in enumerate(idx):
        e = ex[k]
        if p.prec == "w":
            v = Fraction(float(x_out[i, 0])) + Fraction(float(x_out[i, 1]))
            errs[k] = abs(float(v - e))
        elif p.prec in ("c", "z"):
            errs[k] = abs(complex(float(_frac(x_out[i].real) - e[0]),
                                  float(_frac(x_out[i].imag) - e[1])))
        else:
            errs[k] = abs(float(_frac(x_out[i]) - e))
    return errs


def trmv_tolerance(p, rows=None):
    """4*n*eps*(|op(T)||x|)_i for all outputs (logical order), or for the
    outputs ``rows`` only (unit increment, read without forming op(T))."""
    n = max(p.n, 1)
    if rows is None:
        x = _magnitude(p, p.x[vec_index(p.n, p.incx)])
        t = np.abs(trmv_op_dense(p)) @ x
    else:
        assert p.incx == 1
        rows = np.asarray(rows, dtype=np.int64)
        x = _magnitude(p, p.x)
        up = is_upper(p.uplo)
        tr = p.trans not in ("N", "n")
        t = np.empty(len(rows))
        for q, o in enumerate(rows):
            # stored entries of row o of op(T): column o of T when transposed
            if tr:
                ks = np.arange(0, o + 1) if up else np.arange(o, p.n)
                idx = ks + o * p.lda
            else:
                ks = np.arange(o, p.n) if up else np.arange(0, o + 1)
                idx = o + ks * p.lda
            mag = _magnitude(p, p.A[idx])
            if _trmv_unit(p):
                mag[ks == o] = 1.0
            t[q] = float(mag @ x[ks])
    return 4.0 * n * EPS[p.prec] * t


def trmv_integer_expected(p):
    """Exact op(T)*x of an integer-valued TrmvProblem via int64 products, in
    the element type (logical order)."""
    M = trmv_op_dense(p)
    xi = vec_index(p.n, p.incx)
    if p.prec in ("c", "z"):
        Mr = np.rint(M.real).astype(np.int64)
        Mi = np.rint(M.imag).astype(np.int64)
        xr = np.rint(p.x[xi].real).astype(np.int64)
        xim = np.rint(p.x[xi].imag).astype(np.int64)
        s = (Mr @ xr - Mi @ xim).astype(np.complex128) + 1j * (Mr @ xim + Mi @ xr)
        return s.astype(p.x.dtype)
    Mi = np.rint(M).astype(np.int64)
    if p.prec == "w":
        r = np.zeros((p.n, 2))
        r[:, 0] = (Mi @ np.rint(p.x[xi, 0]).astype(np.int64)).astype(np.float64)
        return r
    return (Mi @ np.rint(p.x[xi]).astype(np.int64)).astype(p.x.dtype)


# ------------------------------------------------- sharded product (one GPU's share)

def panel_owner_def(q: int, nshards: int) -> int:
    """Shard owning panel q: rounds of nshards panels, dealt forward in even
    rounds and backward in odd ones."""
    rnd, pos = divmod(q, nshards)
    return pos if rnd % 2 == 0 else nshards - 1 - pos


def shard_columns_def(n: int, panel: int, nshards: int, shard: int) -> np.ndarray:
    return np.array([j for j in range(n) if panel_owner_def(j // panel, nshards) == shard],
                    dtype=np.int64)


def local_matrix(p, cols) -> np.ndarray:
    """The shard's local matrix: columns ``cols`` of A (all lda rows each),
    in order."""
    lda = p.lda
    idx = (np.asarray(cols, dtype=np.int64)[:, None] * lda +
           np.arange(lda, dtype=np.int64)[None, :]).reshape(-1)
    return np.ascontiguousarray(p.A[idx])


def shard_exact(p, nshards, panel, shard):
    """Exact partial of a shard, row by row over the full symmetric S: entry
    S(i,j) belongs to the shard owning the column of the stored element that
    represents it ((i,j) if stored, else (j,i))."""
    n = p.n
    get = exact_elements(p)
    cplx = p.prec in ("c", "z")
    x = exact_vector(p, p.x, p.incx)
    zero = (Fraction(0), Fraction(0)) if cplx else Fraction(0)
    out = []
    for i in range(n):
        s = zero
        for j in range(n):
            col = j if stored(p.uplo, i, j) else i
            if panel_owner_def(col // panel, nshards) != shard:
                continue
            if i == j:
                a = get(i, i)
                if cplx:
                    a = (a[0], Fraction(0))
            elif stored(p.uplo, i, j):
                a = get(i, j)
            else:
                a = get(j, i)
                if cplx:
                    a = (a[0], -a[1])
            s = _cadd(s, _cmul(a, x[j])) if cplx else s + a * x[j]
        out.append(s)
    return out


def shard_mask(p, nshards, panel, shard) -> np.ndarray:
    """0/1 mask of the entries of S that belong to the shard."""
    n = p.n
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    st = (i <= j) if is_upper(p.uplo) else (i >= j)
    col = np.where(st, j, i)
    own = np.array([panel_owner_def(c // panel, nshards) for c in range(n)])
    return own[col] == shard


def shard_tolerance(p, nshards, panel, shard):
    """4*n*eps*(|S_g||x|)_i, S_g the shard's entries of S."""
    M = np.abs(dense_matrix(p)) * shard_mask(p, nshards, panel, shard)
    x = _magnitude(p, p.x[vec_index(p.n, p.incx)])
    return 4.0 * max(p.n, 1) * EPS[p.prec] * (M @ x)


def exact_value_errors(prec, got, exact):
    """|got_k - exact_k| for a contiguous vector against exact values."""
    errs = np.empty(len(exact))
    for k, e in enumerate(exact):
        if prec == "w":
            v = Fraction(float(got[k, 0])) + Fraction(float(got[k, 1]))
            errs[k] = abs(float(v - e))
        elif prec in ("c", "z"):
            errs[k] = abs(complex(float(_frac(got[k].real) - e[0]),
                                  float(_frac(got[k].imag) - e[1])))
        else:
            errs[k] = abs(float(_frac(got[k]) - e))
    return errs
