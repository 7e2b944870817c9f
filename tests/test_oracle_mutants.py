"""The pins have teeth: plant plausible mistakes in a copy of the oracle's
source (on the CPU only), build each copy, and check that the pin battery of
``test_oracle_pins`` rejects every one of them.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_gemv as G
from tests import test_oracle_syr2 as R2
from tests import test_oracle_trmv as TM
from tests import test_oracle_shard as SH
from tests import test_oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "xsymv_oracle.c")

# (name, text in the oracle, replacement, occurrence to change or None = all)
MUTANTS = [
    ("mirrored element not conjugated",
     "return P##_conj(A[j + i * lda]);", "return A[j + i * lda];", None),
    ("mirrored element read from the unstored triangle",
     "return P##_conj(A[j + i * lda]);", "return P##_conj(A[i + j * lda]);", None),
    ("stored element read transposed",
     "if (upper ? (i < j) : (i > j)) return A[i + j * lda];",
     "if (upper ? (i < j) : (i > j)) return A[j + i * lda];", None),
    ("triangles swapped",
     "if (upper ? (i < j) : (i > j)) return", "if (upper ? (i > j) : (i < j)) return", None),
    ("diagonal dropped",
     "if (i == j) return P##_diag(&A[i + i * lda]);", "if (i == j) return P##_zero();", None),
    ("x(i) in place of x(j)",
     "sum = P##_add(sum, P##_mul(s, x[vpos(n, incx, j)]));",
     "sum = P##_add(sum, P##_mul(s, x[vpos(n, incx, (int)i)]));", 1),
    ("inner sum one term short",
     "for (j = 0; j < n; ++j) {", "for (j = 0; j < n - 1; ++j) {", 1),
    ("beta = 0 multiplies y",
     "T res = P##_is_zero(beta) ? P##_zero() : P##_mul(beta, *yi);",
     "T res = P##_mul(beta, *yi);", 1),
    ("alpha dropped",
     "res = P##_add(res, P##_mul(alpha, sum));", "res = P##_add(res, sum);", None),
    ("Hermitian diagonal keeps the imaginary word (single)",
     "r.im = 0.0f;", "r.im = p->im;", 1),
    ("Hermitian diagonal keeps the imaginary word (double)",
     "r.im = 0.0;\n    return r;\n}\nstatic int z_is_zero",
     "r.im = p->im;\n    return r;\n}\nstatic int z_is_zero", None),
    ("complex product sign",
     "r.re = a.re * b.re - a.im * b.im;", "r.re = a.re * b.re + a.im * b.im;", 1),
    ("double complex product sign",
     "r.re = a.re * b.re - a.im * b.im;", "r.re = a.re * b.re + a.im * b.im;", 2),
    ("sloppy double-double add",
     "    s.lo = s.lo + t.hi;\n    s = fast_two_sum(s.hi, s.lo);\n    s.lo = s.lo + t.lo;",
     "    s.lo = s.lo + (a.lo + b.lo);", None),
    ("double-double product drops cross terms",
     "p.lo = p.lo + (a.hi * b.lo + a.lo * b.hi);", "p.lo = p.lo;", None),
    ("TwoProd without its error term",
     "r.lo = fma(a, b, -p);", "r.lo = 0.0;", None),
    ("increments ignored",
     "return start + (long long)k * inc;", "return (long long)k;", None),
    ("gemv: 'N' reads the transposed element",
     "T a = tr == 0 ? A[(long long)o + (long long)k * lda]",
     "T a = tr == 0 ? A[(long long)k + (long long)o * lda]", None),
    ("gemv: 'C' without conjugate",
     "if (tr == 2) a = P##_conj(a);", "(void)0;", None),
    ("gemv: beta = 0 multiplies y",
     "T res = P##_is_zero(beta) ? P##_zero() : P##_mul(beta, *yi);",
     "T res = P##_mul(beta, *yi);", 2),
    ("gemv: alpha dropped",
     "res = P##_add(res, P##_mul(alpha, P##_gemv_dot(",
     "res = P##_add(res, (P##_gemv_dot(", 1),
    ("gemv: inner loop one short",
     "for (k = 0; k < kl; ++k) {", "for (k = 0; k < kl - 1; ++k) {", None),
    ("syr2: t2 built from y",
     "T t2 = HERM ? P##_conj(P##_mul(alpha, xj)) : P##_mul(alpha, xj);",
     "T t2 = HERM ? P##_conj(P##_mul(alpha, yj)) : P##_mul(alpha, yj);", None),
    ("her2: t1 without conjugate",
     "T t1 = P##_mul(alpha, HERM ? P##_conj(yj) : yj);",
     "T t1 = P##_mul(alpha, yj);", None),
    ("her2: diagonal keeps its imaginary part",
     "r.re = a.re + s.re;\n    r.im = 0.0f;", "r.re = a.re + s.re;\n    r.im = a.im;", None),
    ("syr2: lower update also writes the diagonal's upper neighbour",
     "int lo = upper ? 0 : j, hi = upper ? j + 1 : n;",
     "int lo = upper ? 0 : (j > 0 ? j - 1 : 0), hi = upper ? j + 1 : n;", None),
    ("syr2: upper update skips the diagonal",
     "int lo = upper ? 0 : j, hi = upper ? j + 1 : n;",
     "int lo = upper ? 0 : j, hi = upper ? j : n;", None),
    ("trmv: the other triangle",
     "if (upper ? r > c : r < c) continue;", "if (upper ? r < c : r > c) continue;", None),
    ("trmv: diagonal skipped",
     "if (upper ? r > c : r < c) continue;", "if (upper ? r >= c : r <= c) continue;", None),
    ("trmv: 'N' and 'T' indices swapped",
     "int r = tr == 0 ? i : k, c = tr == 0 ? k : i;",
     "int r = tr == 0 ? k : i, c = tr == 0 ? i : k;", None),
    ("trmv: 'C' without conjugate",
     "a = A[(long long)r + (long long)c * lda];",
     "a = A[(long long)r + (long long)c * lda]; tr = tr == 2 ? 1 : tr;", None),
    ("trmv: unit diagonal read from A",
     "if (r == c && unit) {", "if (0 && unit) {", None),
    ("trmv: x overwritten while outputs are formed",
     "out[i] = sum;", "out[i] = sum; x[vpos(n, incx, i)] = sum;", None),
    ("shard: panels dealt cyclically, not back and forth",
     "return round % 2 == 0 ? pos : nshards - 1 - pos;", "(void)round; return pos;", None),
    ("shard: mirrored terms dropped",
     "s = stored_here ? *ap : P##_conj(*ap);",
     "if (!stored_here) continue; s = *ap;", None),
    ("shard: mirrored terms without conjugate",
     "s = stored_here ? *ap : P##_conj(*ap);", "s = *ap;", None),
    ("shard: diagonal counted twice",
     "s = P##_diag(ap);", "s = P##_add(P##_diag(ap), P##_diag(ap));", None),
    ("shard: local column index not advanced",
     "== shard ? l++ : -1;", "== shard ? l : -1;", None),
    ("shard: mirrored term owned by column j",
     "int col = stored_here ? j : i, row", "int col = j, row", None),
    ("combine: partials summed out of rank order",
     "for (g = 1; g < nshards; ++g)", "for (g = nshards - 1; g >= 1; --g)", None),
    ("combine: beta = 0 multiplies y",
     "T r = P##_is_zero(beta) ? P##_zero() : P##_mul(beta, *yi);",
     "T r = P##_mul(beta, *yi);", None),
    ("gemv: x walked with y's increment",
     "sum = P##_add(sum, P##_mul(a, x[vpos(lenx, incx, k)]));",
     "sum = P##_add(sum, P##_mul(a, x[vpos(lenx, 1, k)]));", None),
]

# pin battery: (test function, parameter sets)
BATTERY = [
    (P.test_exact_bruteforce, [dict(prec=pr, uplo=u, n=17, pad=3)
                               for pr in P.PRECS for u in "LU"]),
    (P.test_integer_inputs_bitwise, [dict(prec=pr, uplo=u, n=64, pad=5)
                                     for pr in P.PRECS for u in "LU"]),
    (P.test_hermitian_diagonal_imaginary_ignored, [dict(prec=pr, uplo=u)
                                                   for pr in "cz" for u in "LU"]),
    (P.test_beta_zero_ignores_nan_y, [dict(prec=pr) for pr in P.PRECS]),
    (P.test_increments, [dict(prec=pr, incx=-3, incy=-2) for pr in P.PRECS]),
    (P.test_dd_add_mul_exact_cases, [dict()]),
    (P.test_dd_add_mul_relative_error, [dict()]),
    (G.test_gemv_exact_bruteforce, [dict(prec=pr, trans=t, m=13, n=11, pad=3)
                                    for pr in G.PRECS for t in G.TRANS]),
    (G.test_gemv_integer_bitwise, [dict(prec=pr, trans=t, m=64, n=48, pad=5)
                                   for pr in G.PRECS for t in G.TRANS]),
    (G.test_gemv_beta_zero_ignores_nan_y, [dict(prec=pr, trans=t)
                                           for pr in G.PRECS for t in "NT"]),
    (G.test_gemv_increments, [dict(prec=pr, trans="N", incx=2, incy=-3) for pr in G.PRECS]),
    (R2.test_syr2_exact_bruteforce, [dict(prec=pr, uplo=u, n=6, pad=2)
                                     for pr in R2.PRECS for u in "LU"]),
    (R2.test_syr2_other_triangle_and_padding_untouched, [dict(prec=pr, uplo=u)
                                                         for pr in R2.PRECS for u in "LU"]),
    (R2.test_her2_diagonal_real, [dict(prec=pr, uplo=u) for pr in "cz" for u in "LU"]),
    (TM.test_trmv_exact_bruteforce, [dict(prec=pr, uplo=u, trans=t, diag=d, n=7, pad=2)
                                     for pr in TM.PRECS for u in "LU" for t in TM.TRANS
                                     for d in "NU"]),
    (TM.test_trmv_unit_diagonal_not_read, [dict(prec=pr, uplo=u, trans=t)
                                           for pr in TM.PRECS for u in "LU" for t in TM.TRANS]),
    (SH.test_shard_columns_definition, [dict(n=37, panel=4, nshards=3)]),
    (SH.test_shard_exact_bruteforce, [dict(prec=pr, uplo=u, n=13, pad=1, panel=2, nshards=4)
                                      for pr in SH.PRECS for u in "LU"]),
    (SH.test_combine_sums_in_rank_order, [dict()]),
    (SH.test_combine_zero_scalars, [dict(prec=pr) for pr in SH.PRECS]),
]


def build_mutant(tmp_path, old, new, occurrence):
    src = open(SRC).read()
    assert old in src, f"mutation anchor not found: {old!r}"
    if occurrence is None:
        mutated = src.replace(old, new)
    else:
        parts = src.split(old)
        assert len(parts) > occurrence
        mutated = old.join(parts[:occurrence]) + new + old.join(parts[occurrence:])
    assert mutated != src
    c = tmp_path / "mutant.c"
    c.write_text(mutated)
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", *oracle.CFLAGS, "-I", os.path.dirname(SRC), "-o", str(so),
                    str(c), "-lm"], check=True, capture_output=True)
    return oracle.OracleLib(str(so))


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(name, old, new, occ, tmp_path):
    lib = build_mutant(tmp_path, old, new, occ)
    for fn, params in BATTERY:
        for kw in params:
            try:
                fn(oracle_lib=lib, **kw)
            except (AssertionError, ValueError):
                return  # killed
    pytest.fail(f"no pin rejects the mutant '{name}'")


def test_unmutated_copy_passes(tmp_path):
    """The battery itself passes on an unmodified copy of the oracle."""
    lib = oracle.OracleLib(oracle.default().path)
    for fn, params in BATTERY:
        for kw in params:
            fn(oracle_lib=lib, **kw)
