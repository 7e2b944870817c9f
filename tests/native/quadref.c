/*
 * quadref.c -- test checker: rows of alpha*S*x + beta*y evaluated in binary128
 * (__float128, 113-bit significand), from the definition of the product
 * (CUDA-xSYMV report, §1 eq.(1)) on the explicitly mirrored matrix.
 *
 * Independent of the oracle and of the GPU library.  Inputs are double or
 * double-double (hi, lo) arrays, unit increments, column-major A.  Each
 * result is returned as the pair (hi, lo) = (RN(q), RN(q - hi)), which keeps
 * about 106 bits of the binary128 value.
 */
#include <stddef.h>

typedef __float128 q_t;

static q_t dd_in(const double *p) { return (q_t)p[0] + (q_t)p[1]; }

static int stored(int upper, long long i, long long j)
{
    return upper ? (i <= j) : (i >= j);
}

static void out2(q_t q, double *hi, double *lo)
{
    double h = (double)q;
    *hi = h;
    *lo = (double)(q - (q_t)h);
}

/* elem_words = 1 (double) or 2 (double-double) */
static int rows_q(int elem_words, char uplo, int n, const double *alpha,
                  const double *A, int lda, const double *x, const double *beta,
                  const double *y, const long long *rows, int nrows,
                  double *out_hi, double *out_lo)
{
    int upper = (uplo == 'U' || uplo == 'u');
    q_t al = elem_words == 2 ? dd_in(alpha) : (q_t)alpha[0];
    q_t be = elem_words == 2 ? dd_in(beta) : (q_t)beta[0];
    for (int r = 0; r < nrows; ++r) {
        long long i = rows[r];
        q_t s = 0;
        if (i < 0 || i >= n) return -1;
        for (long long j = 0; j < n; ++j) {
            long long k = stored(upper, i, j) ? i + j * (long long)lda
                                              : j + i * (long long)lda;
            const double *a = A + k * elem_words;
            const double *xj = x + j * elem_words;
            q_t av = elem_words == 2 ? dd_in(a) : (q_t)a[0];
            q_t xv = elem_words == 2 ? dd_in(xj) : (q_t)xj[0];
            s += av * xv;
        }
        q_t res = al * s;
        if (be != 0) {
            const double *yi = y + i * elem_words;
            res += be * (elem_words == 2 ? dd_in(yi) : (q_t)yi[0]);
        }
        out2(res, &out_hi[r], &out_lo[r]);
    }
    return 0;
}

int quad_wsymv_rows(char uplo, int n, const double *alpha, const double *A,
                    int lda, const double *x, const double *beta,
                    const double *y, const long long *rows, int nrows,
                    double *out_hi, double *out_lo)
{
    return rows_q(2, uplo, n, alpha, A, lda, x, beta, y, rows, nrows,
                  out_hi, out_lo);
}

int quad_dsymv_rows(char uplo, int n, const double *alpha, const double *A,
                    int lda, const double *x, const double *beta,
                    const double *y, const long long *rows, int nrows,
                    double *out_hi, double *out_lo)
{
    return rows_q(1, uplo, n, alpha, A, lda, x, beta, y, rows, nrows,
                  out_hi, out_lo);
}

/* Output elements rows[] of alpha*op(A)*x + beta*y for a general m x n A
 * (op = A for trans 'N', A^T otherwise), double-double or double inputs, unit
 * increments; from the definition, in binary128. */
static int gemv_q(int elem_words, char trans, int m, int n, const double *alpha,
                  const double *A, int lda, const double *x, const double *beta,
                  const double *y, const long long *rows, int nrows,
                  double *out_hi, double *out_lo)
{
    int tr = !(trans == 'N' || trans == 'n');
    long long leny = tr ? n : m, lenx = tr ? m : n;
    q_t al = elem_words == 2 ? dd_in(alpha) : (q_t)alpha[0];
    q_t be = elem_words == 2 ? dd_in(beta) : (q_t)beta[0];
    for (int r = 0; r < nrows; ++r) {
        long long o = rows[r];
        q_t s = 0;
        if (o < 0 || o >= leny) return -1;
        for (long long k = 0; k < lenx; ++k) {
            long long idx = tr ? k + o * (long long)lda : o + k * (long long)lda;
            const double *a = A + idx * elem_words;
            const double *xk = x + k * elem_words;
            q_t av = elem_words == 2 ? dd_in(a) : (q_t)a[0];
            q_t xv = elem_words == 2 ? dd_in(xk) : (q_t)xk[0];
            s += av * xv;
        }
        q_t res = al * s;
        if (be != 0) {
            const double *yo = y + o * elem_words;
            res += be * (elem_words == 2 ? dd_in(yo) : (q_t)yo[0]);
        }
        out2(res, &out_hi[r], &out_lo[r]);
    }
    return 0;
}

int quad_wgemv_rows(char trans, int m, int n, const double *alpha, const double *A,
                    int lda, const double *x, const double *beta, const double *y,
                    const long long *rows, int nrows, double *out_hi, double *out_lo)
{
    return gemv_q(2, trans, m, n, alpha, A, lda, x, beta, y, rows, nrows, out_hi, out_lo);
}

int quad_dgemv_rows(char trans, int m, int n, const double *alpha, const double *A,
                    int lda, const double *x, const double *beta, const double *y,
                    const long long *rows, int nrows, double *out_hi, double *out_lo)
{
    return gemv_q(1, trans, m, n, alpha, A, lda, x, beta, y, rows, nrows, out_hi, out_lo);
}
