/*
 * xsymv_oracle.c -- CPU oracle for the symmetric / Hermitian matrix-vector
 * product y := alpha*S*x + beta*y in five element types.
 *
 * TEST INFRASTRUCTURE ONLY: called by the test suite, the packaged smoke
 * check and the benchmark's CPU-baseline leg, never by the product path.
 * It shares no source with the GPU library (no common headers, helpers or
 * tables).  Build: gcc -O2 -ffp-contract=off -std=c99 -fPIC -shared -lm, so
 * that every product and sum is rounded exactly as written (no contraction
 * into fused multiply-adds except where fma() is called by name).
 *
 * What it computes.  The CUDA-xSYMV report (IPSJ SIG Technical Report
 * 2014-HPC-146 No.14), §1 eq.(1): y := alpha*A_{U or L}*x + beta*y with
 * A = A^T, where only the upper (U) or lower (L) triangle is stored and
 * referenced.  S below is the full matrix that triangle implies:
 *   S(i,j) = A(i,j) where (i,j) is stored, conj(A(j,i)) across the diagonal,
 *   and for Hermitian matrices S(i,i) = Re A(i,i) (the imaginary word of a
 *   diagonal element is never read).  conj() is the identity for the real
 *   and double-double types.
 *
 * How.  The definition written out, one output element at a time:
 *   y(i) := beta*y(i) + alpha * sum over j = 0, 1, ..., n-1 of S(i,j)*x(j),
 * the inner index ascending, in the working precision.  Each output reads
 * only its own y(i), so y is overwritten in place.  The BLAS rules hold:
 * with beta == 0 the old y is not read (it may hold NaN), alpha == 0 leaves
 * y := beta*y without touching A or x, and n == 0 or (alpha == 0 and
 * beta == 1) returns at once.  Outputs are independent, so the full product
 * may be spread over threads (oracle_set_threads; OpenMP) with the same bits
 * for any thread count.
 *
 * General matrix-vector product (the report's point of comparison: SYMV
 * reads one triangle, GEMV the whole matrix, §1 and §2.1), BLAS xGEMV:
 *   y := alpha*op(A)*x + beta*y, op(A) = A ('N'), A^T ('T') or A^H ('C'),
 * A m x n column-major.  Written out from the definition, one output element
 * at a time: y(i) := beta*y(i) + alpha * sum over the inner index k,
 * ascending, of op(A)(i,k)*x(k), in the working precision.  Same BLAS rules
 * for beta == 0 (y not read), alpha == 0 and the quick return.
 *
 * Symmetric / Hermitian rank-2 update (the report's §5 extends the approach
 * to other Level-2 BLAS), BLAS xSYR2 / xHER2 on the stored triangle:
 *   A := alpha*x*y^H + conj(alpha)*y*x^H + A  (real: alpha*x*y^T + alpha*y*x^T)
 * in the BLAS reference order: for each column j, t1 = alpha*conj(y(j)),
 * t2 = conj(alpha*x(j)), and every stored A(i,j) := (A(i,j) + x(i)*t1) +
 * y(i)*t2; a Hermitian diagonal element becomes Re(A(j,j)) +
 * Re(x(j)*t1 + y(j)*t2) with a zero imaginary part.  The other triangle is
 * neither read nor written.
 *
 * Triangular matrix-vector product (another of the Level-2 BLAS the
 * report's §5 points to), BLAS xTRMV: x := op(T)*x with T the stored
 * triangle of A (diagonal from A, or 1 for a unit triangle -- then the
 * diagonal is not read), op = T, T^T or T^H.  Each output element from the
 * definition: the sum over the inner index k ascending of op(T)(i,k)*x(k),
 * in the working precision; all outputs are formed before x is overwritten.
 *
 * One GPU's share of the product (the path sharded over several GPUs with
 * one exchange; the report's §5 points to multi-GPU SYMV, ref. [7]).  The
 * columns are cut into panels of `panel` consecutive columns (the last one
 * may be short); the panels are dealt to `nshards` shards round by round, in
 * even rounds shard g taking the round's g-th panel and in odd rounds its
 * (nshards-1-g)-th (boustrophedon order, so the shards' triangle areas stay
 * close).  A shard keeps only its own columns, in ascending order, as a local
 * column-major matrix.  Its partial vector holds, for every output i, the
 * terms S(i,j)*x(j) (j ascending) whose element S(i,j) is stored in one of
 * its columns -- column j when (i,j) is in the stored triangle, column i
 * otherwise -- so that every term of S*x belongs to exactly one shard and the
 * shards' partials add up to S*x.  The exchange then gives every
 * GPU all partials, and y(i) := beta*y(i) + alpha*(p_0(i) + p_1(i) + ...),
 * summed in rank order (the report's fixed summation order, §2.1, kept
 * across GPUs), with the BLAS rules for beta == 0 and alpha == 0.
 *
 * Double-double arithmetic (report §2.2, which takes Bailey's double-double
 * format [14]: a value is the unevaluated sum hi + lo of two doubles):
 *   TwoSum (Knuth) and FastTwoSum (Dekker) give a sum and its exact error;
 *   TwoProd gives a product and its exact error with one fma;
 *   dd_add is the accurate ("IEEE") double-double addition of Hida, Li and
 *     Bailey -- both hi and lo parts are summed with TwoSum and the result
 *     is renormalised twice;
 *   dd_mul is their multiplication: TwoProd of the high parts plus the two
 *     cross products, then renormalised.
 */
#include "xsymv_oracle.h"

#include <math.h>
#include <stdlib.h>

/* ----------------------------------------------------------------- checks */

/* BLAS argument checks, in the order of the report's argument list
 * (§2.2 Fig. 5: uplo, n, alpha, a, lda, x, incx, beta, y, incy). */
static int check_args(char uplo, int n, const void *A, int lda,
                      const void *x, int incx, const void *y, int incy,
                      int *upper)
{
    if (uplo == 'U' || uplo == 'u')
        *upper = 1;
    else if (uplo == 'L' || uplo == 'l')
        *upper = 0;
    else
        return -1;
    if (n < 0) return -2;
    if (n > 0 && A == NULL) return -4;
    if (lda < (n > 1 ? n : 1)) return -5;
    if (n > 0 && x == NULL) return -6;
    if (incx == 0) return -7;
    if (n > 0 && y == NULL) return -9;
    if (incy == 0) return -10;
    return 0;
}

/* Position of logical element k of a strided vector (BLAS convention). */
static long long vpos(int n, int inc, int k)
{
    long long start = inc > 0 ? 0 : (long long)(1 - n) * inc;
    return start + (long long)k * inc;
}

/* ------------------------------------------------------- element types */

/* real single */
static float s_add(float a, float b) { return a + b; }
static float s_mul(float a, float b) { return a * b; }
static float s_conj(float a) { return a; }
static float s_diag(const float *p) { return *p; }
static int s_is_zero(float a) { return a == 0.0f; }
static int s_is_one(float a) { return a == 1.0f; }
static float s_zero(void) { return 0.0f; }

/* real double */
static double d_add(double a, double b) { return a + b; }
static double d_mul(double a, double b) { return a * b; }
static double d_conj(double a) { return a; }
static double d_diag(const double *p) { return *p; }
static int d_is_zero(double a) { return a == 0.0; }
static int d_is_one(double a) { return a == 1.0; }
static double d_zero(void) { return 0.0; }

/* complex single: textbook product, four products and two sums */
static ocplx_f c_add(ocplx_f a, ocplx_f b)
{
    ocplx_f r;
    r.re = a.re + b.re;
    r.im = a.im + b.im;
    return r;
}
static ocplx_f c_mul(ocplx_f a, ocplx_f b)
{
    ocplx_f r;
    r.re = a.re * b.re - a.im * b.im;
    r.im = a.re * b.im + a.im * b.re;
    return r;
}
static ocplx_f c_conj(ocplx_f a)
{
    a.im = -a.im;
    return a;
}
/* Hermitian diagonal: only the real word is read. */
static ocplx_f c_diag(const ocplx_f *p)
{
    ocplx_f r;
    r.re = p->re;
    r.im = 0.0f;
    return r;
}
static int c_is_zero(ocplx_f a) { return a.re == 0.0f && a.im == 0.0f; }
static int c_is_one(ocplx_f a) { return a.re == 1.0f && a.im == 0.0f; }
static ocplx_f c_zero(void)
{
    ocplx_f r = {0.0f, 0.0f};
    return r;
}

/* complex double */
static ocplx_d z_add(ocplx_d a, ocplx_d b)
{
    ocplx_d r;
    r.re = a.re + b.re;
    r.im = a.im + b.im;
    return r;
}
static ocplx_d z_mul(ocplx_d a, ocplx_d b)
{
    ocplx_d r;
    r.re = a.re * b.re - a.im * b.im;
    r.im = a.re * b.im + a.im * b.re;
    return r;
}
static ocplx_d z_conj(ocplx_d a)
{
    a.im = -a.im;
    return a;
}
static ocplx_d z_diag(const ocplx_d *p)
{
    ocplx_d r;
    r.re = p->re;
    r.im = 0.0;
    return r;
}
static int z_is_zero(ocplx_d a) { return a.re == 0.0 && a.im == 0.0; }
static int z_is_one(ocplx_d a) { return a.re == 1.0 && a.im == 0.0; }
static ocplx_d z_zero(void)
{
    ocplx_d r = {0.0, 0.0};
    return r;
}

/* double-double */
static odd two_sum(double a, double b)          /* Knuth: any a, b */
{
    odd r;
    double s = a + b;
    double bb = s - a;
    r.hi = s;
    r.lo = (a - (s - bb)) + (b - bb);
    return r;
}
static odd fast_two_sum(double a, double b)     /* Dekker: |a| >= |b| */
{
    odd r;
    double s = a + b;
    r.hi = s;
    r.lo = b - (s - a);
    return r;
}
static odd two_prod(double a, double b)         /* exact via one fma */
{
    odd r;
    double p = a * b;
    r.hi = p;
    r.lo = fma(a, b, -p);
    return r;
}
odd oracle_dd_add(odd a, odd b)
{
    odd s = two_sum(a.hi, b.hi);
    odd t = two_sum(a.lo, b.lo);
    s.lo = s.lo + t.hi;
    s = fast_two_sum(s.hi, s.lo);
    s.lo = s.lo + t.lo;
    return fast_two_sum(s.hi, s.lo);
}
odd oracle_dd_mul(odd a, odd b)
{
    odd p = two_prod(a.hi, b.hi);
    p.lo = p.lo + (a.hi * b.lo + a.lo * b.hi);
    return fast_two_sum(p.hi, p.lo);
}
static odd w_add(odd a, odd b) { return oracle_dd_add(a, b); }
static odd w_mul(odd a, odd b) { return oracle_dd_mul(a, b); }
static odd w_conj(odd a) { return a; }
static odd w_diag(const odd *p) { return *p; }
static int w_is_zero(odd a) { return a.hi == 0.0 && a.lo == 0.0; }
static int w_is_one(odd a) { return a.hi == 1.0 && a.lo == 0.0; }
static odd w_zero(void)
{
    odd r = {0.0, 0.0};
    return r;
}

/* ------------------------------------------------------------ algorithm */

/* Threads the full-product entry points use (rows are independent, so any
 * count gives the same bits); 1 unless set. */
static int g_threads = 1;

int oracle_set_threads(int nthreads)
{
    if (nthreads < 1) return -1;
#ifdef _OPENMP
    g_threads = nthreads;
#else
    if (nthreads > 1) return -2;
#endif
    return 0;
}

int oracle_get_threads(void) { return g_threads; }

/* One definition per element type; P is the prefix of its operations.
 *
 * elem: S(i,j), the element of the full matrix that the stored triangle
 *   implies -- A(i,j) where (i,j) is stored, conj(A(j,i)) across the
 *   diagonal, and on the diagonal its stored value (Hermitian: the real word
 *   alone).
 * row: output i of eq.(1), beta*Y(i) + alpha * sum over j = 0, 1, ..., n-1
 *   (ascending) of S(i,j)*X(j); with beta == 0 the old Y(i) is not read,
 *   with alpha == 0 neither A nor x is. */
#define DEFINE_ORACLE(NAME, ROWS_NAME, T, P)                                   \
static T P##_elem(int upper, const T *A, int lda, long long i, long long j)    \
{                                                                              \
    if (i == j) return P##_diag(&A[i + i * lda]);                              \
    if (upper ? (i < j) : (i > j)) return A[i + j * lda];                      \
    return P##_conj(A[j + i * lda]);                                           \
}                                                                              \
                                                                               \
static T P##_row(int upper, int n, T alpha, const T *A, int lda, const T *x,   \
                 int incx, T beta, const T *yi, long long i)                   \
{                                                                              \
    int j;                                                                     \
    T res = P##_is_zero(beta) ? P##_zero() : P##_mul(beta, *yi);               \
    if (!P##_is_zero(alpha)) {                                                 \
        T sum = P##_zero();                                                    \
        for (j = 0; j < n; ++j) {                                              \
            T s = P##_elem(upper, A, lda, i, j);                               \
            sum = P##_add(sum, P##_mul(s, x[vpos(n, incx, j)]));               \
        }                                                                      \
        res = P##_add(res, P##_mul(alpha, sum));                               \
    }                                                                          \
    return res;                                                                \
}                                                                              \
                                                                               \
int NAME(char uplo, int n, T alpha, const T *A, int lda, const T *x,           \
         int incx, T beta, T *y, int incy)                                     \
{                                                                              \
    int upper, i;                                                              \
    int rc = check_args(uplo, n, A, lda, x, incx, y, incy, &upper);            \
    if (rc) return rc;                                                         \
    if (n == 0 || (P##_is_zero(alpha) && P##_is_one(beta))) return 0;          \
    /* output i reads Y(i) alone, so y is updated in place row by row */       \
    _Pragma("omp parallel for schedule(dynamic, 16) num_threads(g_threads)")   \
    for (i = 0; i < n; ++i) {                                                  \
        T *yi = &y[vpos(n, incy, i)];                                          \
        *yi = P##_row(upper, n, alpha, A, lda, x, incx, beta, yi, i);          \
    }                                                                          \
    return 0;                                                                  \
}                                                                              \
                                                                               \
int ROWS_NAME(char uplo, int n, T alpha, const T *A, int lda, const T *x,      \
              int incx, T beta, const T *y, int incy, const long long *rows,   \
              int nrows, T *out)                                               \
{                                                                              \
    int upper, r;                                                              \
    int rc = check_args(uplo, n, A, lda, x, incx, y, incy, &upper);            \
    if (rc) return rc;                                                         \
    for (r = 0; r < nrows; ++r)                                                \
        if (rows[r] < 0 || rows[r] >= n) return -11;                           \
    for (r = 0; r < nrows; ++r) {                                              \
        const T *yi = &y[vpos(n, incy, (int)rows[r])];                         \
        out[r] = (P##_is_zero(alpha) && P##_is_one(beta))                      \
                     ? *yi                                                     \
                     : P##_row(upper, n, alpha, A, lda, x, incx, beta, yi,     \
                               rows[r]);                                       \
    }                                                                          \
    return 0;                                                                  \
}

DEFINE_ORACLE(oracle_ssymv, oracle_ssymv_rows, float, s)
DEFINE_ORACLE(oracle_dsymv, oracle_dsymv_rows, double, d)
DEFINE_ORACLE(oracle_chemv, oracle_chemv_rows, ocplx_f, c)
DEFINE_ORACLE(oracle_zhemv, oracle_zhemv_rows, ocplx_d, z)
DEFINE_ORACLE(oracle_wsymv, oracle_wsymv_rows, odd, w)

/* ------------------------------------------------------------- xGEMV */

/* BLAS xGEMV argument checks (xerbla positions: trans, m, n, alpha, a, lda,
 * x, incx, beta, y, incy). */
static int gemv_check(char trans, int m, int n, const void *A, int lda,
                      const void *x, int incx, const void *y, int incy,
                      int *tr)
{
    if (trans == 'N' || trans == 'n')
        *tr = 0;
    else if (trans == 'T' || trans == 't')
        *tr = 1;
    else if (trans == 'C' || trans == 'c')
        *tr = 2;
    else
        return -1;
    if (m < 0) return -2;
    if (n < 0) return -3;
    if (m > 0 && n > 0 && A == NULL) return -5;
    if (lda < (m > 1 ? m : 1)) return -6;
    if (m > 0 && n > 0 && x == NULL) return -7;
    if (incx == 0) return -8;
    if (m > 0 && n > 0 && y == NULL) return -10;
    if (incy == 0) return -11;
    return 0;
}

/* One output element of op(A)*x: output index `o`, inner length `kl`. */
#define DEFINE_GEMV(NAME, ROWS_NAME, T, P)                                      \
static T P##_gemv_dot(int tr, int o, int kl, int lenx, const T *A, int lda,     \
                      const T *x, int incx)                                     \
{                                                                               \
    T sum = P##_zero();                                                         \
    int k;                                                                      \
    for (k = 0; k < kl; ++k) {                                                  \
        T a = tr == 0 ? A[(long long)o + (long long)k * lda]                    \
                      : A[(long long)k + (long long)o * lda];                   \
        if (tr == 2) a = P##_conj(a);                                           \
        sum = P##_add(sum, P##_mul(a, x[vpos(lenx, incx, k)]));                 \
    }                                                                           \
    return sum;                                                                 \
}                                                                               \
                                                                                \
int NAME(char trans, int m, int n, T alpha, const T *A, int lda, const T *x,    \
         int incx, T beta, T *y, int incy)                                      \
{                                                                               \
    int tr, i, leny, lenx;                                                      \
    int rc = gemv_check(trans, m, n, A, lda, x, incx, y, incy, &tr);            \
    if (rc) return rc;                                                          \
    if (m == 0 || n == 0 || (P##_is_zero(alpha) && P##_is_one(beta))) return 0; \
    leny = tr == 0 ? m : n;                                                     \
    lenx = tr == 0 ? n : m;                                                     \
    for (i = 0; i < leny; ++i) {                                                \
        T *yi = &y[vpos(leny, incy, i)];                                        \
        T res = P##_is_zero(beta) ? P##_zero() : P##_mul(beta, *yi);            \
        if (!P##_is_zero(alpha))                                                \
            res = P##_add(res, P##_mul(alpha, P##_gemv_dot(tr, i, lenx, lenx,   \
                                                           A, lda, x, incx)));  \
        *yi = res;                                                              \
    }                                                                           \
    return 0;                                                                   \
}                                                                               \
                                                                                \
int ROWS_NAME(char trans, int m, int n, T alpha, const T *A, int lda,           \
              const T *x, int incx, T beta, const T *y, int incy,               \
              const long long *rows, int nrows, T *out)                         \
{                                                                               \
    int tr, r, leny, lenx;                                                      \
    int rc = gemv_check(trans, m, n, A, lda, x, incx, y, incy, &tr);            \
    if (rc) return rc;                                                          \
    leny = tr == 0 ? m : n;                                                     \
    lenx = tr == 0 ? n : m;                                                     \
    for (r = 0; r < nrows; ++r)                                                 \
        if (rows[r] < 0 || rows[r] >= leny) return -12;                         \
    for (r = 0; r < nrows; ++r) {                                               \
        int i = (int)rows[r];                                                   \
        T yi = y[vpos(leny, incy, i)];                                          \
        T res;                                                                  \
        if (m == 0 || n == 0 || (P##_is_zero(alpha) && P##_is_one(beta))) {     \
            out[r] = yi;                                                        \
            continue;                                                           \
        }                                                                       \
        res = P##_is_zero(beta) ? P##_zero() : P##_mul(beta, yi);               \
        if (!P##_is_zero(alpha))                                                \
            res = P##_add(res, P##_mul(alpha, P##_gemv_dot(tr, i, lenx, lenx,   \
                                                           A, lda, x, incx)));  \
        out[r] = res;                                                           \
    }                                                                           \
    return 0;                                                                   \
}

DEFINE_GEMV(oracle_sgemv, oracle_sgemv_rows, float, s)
DEFINE_GEMV(oracle_dgemv, oracle_dgemv_rows, double, d)
DEFINE_GEMV(oracle_cgemv, oracle_cgemv_rows, ocplx_f, c)
DEFINE_GEMV(oracle_zgemv, oracle_zgemv_rows, ocplx_d, z)
DEFINE_GEMV(oracle_wgemv, oracle_wgemv_rows, odd, w)

/* ------------------------------------------------------- xSYR2 / xHER2 */

/* BLAS xSYR2 / xHER2 argument checks (xerbla positions: uplo, n, alpha, x,
 * incx, y, incy, a, lda). */
static int syr2_check(char uplo, int n, const void *x, int incx, const void *y,
                      int incy, const void *A, int lda, int *upper)
{
    if (uplo == 'U' || uplo == 'u')
        *upper = 1;
    else if (uplo == 'L' || uplo == 'l')
        *upper = 0;
    else
        return -1;
    if (n < 0) return -2;
    if (n > 0 && x == NULL) return -4;
    if (incx == 0) return -5;
    if (n > 0 && y == NULL) return -6;
    if (incy == 0) return -7;
    if (n > 0 && A == NULL) return -8;
    if (lda < (n > 1 ? n : 1)) return -9;
    return 0;
}

/* HERM = 1 for the Hermitian update (complex types): conjugates and the real
 * diagonal; 0 for the symmetric one. */
#define DEFINE_SYR2(NAME, T, P, HERM, REALPART)                                 \
int NAME(char uplo, int n, T alpha, const T *x, int incx, const T *y,          \
         int incy, T *A, int lda)                                               \
{                                                                               \
    int upper, i, j;                                                            \
    int rc = syr2_check(uplo, n, x, incx, y, incy, A, lda, &upper);             \
    if (rc) return rc;                                                          \
    if (n == 0 || P##_is_zero(alpha)) return 0;                                 \
    for (j = 0; j < n; ++j) {                                                   \
        T xj = x[vpos(n, incx, j)], yj = y[vpos(n, incy, j)];                   \
        T t1 = P##_mul(alpha, HERM ? P##_conj(yj) : yj);                        \
        T t2 = HERM ? P##_conj(P##_mul(alpha, xj)) : P##_mul(alpha, xj);        \
        int lo = upper ? 0 : j, hi = upper ? j + 1 : n;                         \
        for (i = lo; i < hi; ++i) {                                             \
            T *a = &A[(long long)i + (long long)j * lda];                       \
            T xi = x[vpos(n, incx, i)], yi = y[vpos(n, incy, i)];               \
            if (HERM && i == j) {                                               \
                T s = P##_add(P##_mul(xi, t1), P##_mul(yi, t2));                \
                *a = REALPART(*a, s);                                           \
            } else {                                                            \
                *a = P##_add(P##_add(*a, P##_mul(xi, t1)), P##_mul(yi, t2));    \
            }                                                                   \
        }                                                                       \
    }                                                                           \
    return 0;                                                                   \
}

/* Re(a) + Re(s), imaginary part zero (the Hermitian diagonal) */
static ocplx_f c_herm_diag(ocplx_f a, ocplx_f s)
{
    ocplx_f r;
    r.re = a.re + s.re;
    r.im = 0.0f;
    return r;
}
static ocplx_d z_herm_diag(ocplx_d a, ocplx_d s)
{
    ocplx_d r;
    r.re = a.re + s.re;
    r.im = 0.0;
    return r;
}
#define NO_REALPART(a, s) ((void)(s), (a))

DEFINE_SYR2(oracle_ssyr2, float, s, 0, NO_REALPART)
DEFINE_SYR2(oracle_dsyr2, double, d, 0, NO_REALPART)
DEFINE_SYR2(oracle_cher2, ocplx_f, c, 1, c_herm_diag)
DEFINE_SYR2(oracle_zher2, ocplx_d, z, 1, z_herm_diag)
DEFINE_SYR2(oracle_wsyr2, odd, w, 0, NO_REALPART)

/* ------------------------------------------------------------- xTRMV */

/* BLAS xTRMV argument checks (xerbla positions: uplo, trans, diag, n, a, lda,
 * x, incx). */
static int trmv_check(char uplo, char trans, char diag, int n, const void *A,
                      int lda, const void *x, int incx, int *upper, int *tr,
                      int *unit)
{
    if (uplo == 'U' || uplo == 'u')
        *upper = 1;
    else if (uplo == 'L' || uplo == 'l')
        *upper = 0;
    else
        return -1;
    if (trans == 'N' || trans == 'n')
        *tr = 0;
    else if (trans == 'T' || trans == 't')
        *tr = 1;
    else if (trans == 'C' || trans == 'c')
        *tr = 2;
    else
        return -2;
    if (diag == 'U' || diag == 'u')
        *unit = 1;
    else if (diag == 'N' || diag == 'n')
        *unit = 0;
    else
        return -3;
    if (n < 0) return -4;
    if (n > 0 && A == NULL) return -5;
    if (lda < (n > 1 ? n : 1)) return -6;
    if (n > 0 && x == NULL) return -7;
    if (incx == 0) return -8;
    return 0;
}

#define DEFINE_TRMV(NAME, T, P)                                                 \
int NAME(char uplo, char trans, char diag, int n, const T *A, int lda, T *x,   \
         int incx)                                                              \
{                                                                               \
    int upper, tr, unit, i, k;                                                  \
    T *out;                                                                     \
    int rc = trmv_check(uplo, trans, diag, n, A, lda, x, incx, &upper, &tr,     \
                        &unit);                                                 \
    if (rc) return rc;                                                          \
    if (n == 0) return 0;                                                       \
    out = (T *)malloc(sizeof(T) * (size_t)n);                                   \
    if (out == NULL) return -100;                                               \
    for (i = 0; i < n; ++i) {                                                   \
        T sum = P##_zero();                                                     \
        for (k = 0; k < n; ++k) {                                               \
            /* op(T)(i,k): element (r, c) of the triangle */                    \
            int r = tr == 0 ? i : k, c = tr == 0 ? k : i;                       \
            T a;                                                                \
            if (upper ? r > c : r < c) continue;  /* outside the triangle */    \
            if (r == c && unit) {                                               \
                sum = P##_add(sum, x[vpos(n, incx, k)]);                        \
                continue;                                                       \
            }                                                                   \
            a = A[(long long)r + (long long)c * lda];                           \
            if (tr == 2) a = P##_conj(a);                                       \
            sum = P##_add(sum, P##_mul(a, x[vpos(n, incx, k)]));                \
        }                                                                       \
        out[i] = sum;                                                           \
    }                                                                           \
    for (i = 0; i < n; ++i) x[vpos(n, incx, i)] = out[i];                       \
    free(out);                                                                  \
    return 0;                                                                   \
}

DEFINE_TRMV(oracle_strmv, float, s)
DEFINE_TRMV(oracle_dtrmv, double, d)
DEFINE_TRMV(oracle_ctrmv, ocplx_f, c)
DEFINE_TRMV(oracle_ztrmv, ocplx_d, z)
DEFINE_TRMV(oracle_wtrmv, odd, w)

/* ------------------------------------------------- one shard's partial */

/* Shard that owns panel q: rounds of nshards panels, boustrophedon order. */
static int panel_owner(int q, int nshards)
{
    int round = q / nshards, pos = q % nshards;
    return round % 2 == 0 ? pos : nshards - 1 - pos;
}

/* Global columns of a shard, ascending; returns their count (cols may be
 * NULL to count only). */
int oracle_shard_columns(int n, int panel, int nshards, int shard, int *cols)
{
    int j, count = 0;
    if (n < 0 || panel <= 0 || nshards <= 0 || shard < 0 || shard >= nshards) return -1;
    for (j = 0; j < n; ++j)
        if (panel_owner(j / panel, nshards) == shard) {
            if (cols) cols[count] = j;
            ++count;
        }
    return count;
}

/* Argument checks: uplo, n, panel, nshards, shard, A, lda, x, incx, p. */
static int shard_check(char uplo, int n, int panel, int nshards, int shard, const void *A,
                       int lda, const void *x, int incx, const void *p, int *upper)
{
    if (uplo == 'U' || uplo == 'u')
        *upper = 1;
    else if (uplo == 'L' || uplo == 'l')
        *upper = 0;
    else
        return -1;
    if (n < 0) return -2;
    if (panel <= 0) return -3;
    if (nshards <= 0) return -4;
    if (shard < 0 || shard >= nshards) return -5;
    if (n > 0 && A == NULL && oracle_shard_columns(n, panel, nshards, shard, NULL) > 0)
        return -6;
    if (lda < (n > 1 ? n : 1)) return -7;
    if (n > 0 && x == NULL) return -8;
    if (incx == 0) return -9;
    if (n > 0 && p == NULL) return -10;
    return 0;
}

/* The shard's share of S*x, from the definition: output i is the sum over
 * j ascending of S(i,j)*X(j) over the j whose S(i,j) is stored in a column
 * the shard owns -- the stored copy of S(i,j) is A(i,j) in column j when
 * (i,j) lies in the stored triangle (the diagonal included), else A(j,i) in
 * column i (conjugated for Hermitian matrices).  Aloc holds owned column c
 * as its local column loc[c], the number of owned columns left of c.  The
 * outputs are independent and may be spread over oracle_set_threads()
 * threads (same bits for any count). */
#define DEFINE_SHARD(NAME, T, P)                                                \
static T P##_shard_row(int upper, int n, const int *loc, const T *Aloc,        \
                       int lda, const T *x, int incx, int i)                   \
{                                                                              \
    int j;                                                                     \
    T sum = P##_zero();                                                        \
    for (j = 0; j < n; ++j) {                                                  \
        int stored_here = upper ? (i <= j) : (i >= j);                         \
        int col = stored_here ? j : i, row = stored_here ? i : j;              \
        const T *ap;                                                           \
        T s;                                                                   \
        if (loc[col] < 0) continue;  /* another shard's column */              \
        ap = &Aloc[(long long)row + (long long)loc[col] * lda];                \
        if (i == j)                                                            \
            s = P##_diag(ap);                                                  \
        else                                                                   \
            s = stored_here ? *ap : P##_conj(*ap);                             \
        sum = P##_add(sum, P##_mul(s, x[vpos(n, incx, j)]));                   \
    }                                                                          \
    return sum;                                                                \
}                                                                              \
                                                                               \
int NAME(char uplo, int n, int panel, int nshards, int shard, const T *Aloc,   \
         int lda, const T *x, int incx, T *p)                                  \
{                                                                              \
    int upper, i, c, l = 0;                                                    \
    int *loc;                                                                  \
    int rc = shard_check(uplo, n, panel, nshards, shard, Aloc, lda, x, incx, p, \
                         &upper);                                              \
    if (rc) return rc;                                                         \
    loc = (int *)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));                \
    if (loc == NULL) return -100;                                              \
    for (c = 0; c < n; ++c)                                                    \
        loc[c] = panel_owner(c / panel, nshards) == shard ? l++ : -1;          \
    _Pragma("omp parallel for schedule(dynamic, 16) num_threads(g_threads)")   \
    for (i = 0; i < n; ++i)                                                    \
        p[i] = P##_shard_row(upper, n, loc, Aloc, lda, x, incx, i);            \
    free(loc);                                                                 \
    return 0;                                                                  \
}

DEFINE_SHARD(oracle_ssymv_shard, float, s)
DEFINE_SHARD(oracle_dsymv_shard, double, d)
DEFINE_SHARD(oracle_chemv_shard, ocplx_f, c)
DEFINE_SHARD(oracle_zhemv_shard, ocplx_d, z)
DEFINE_SHARD(oracle_wsymv_shard, odd, w)

/* y := beta*y + alpha*(P_0 + P_1 + ... ), the partials summed in rank order.
 * Checks: n, nshards, P, ldp, y, incy. */
#define DEFINE_COMBINE(NAME, T, P)                                              \
int NAME(int n, int nshards, T alpha, const T *Pp, int ldp, T beta, T *y,      \
         int incy)                                                             \
{                                                                              \
    int i, g;                                                                  \
    if (n < 0) return -1;                                                      \
    if (nshards <= 0) return -2;                                               \
    if (n > 0 && Pp == NULL) return -4;                                        \
    if (ldp < (n > 1 ? n : 1)) return -5;                                      \
    if (n > 0 && y == NULL) return -7;                                         \
    if (incy == 0) return -8;                                                  \
    if (n == 0 || (P##_is_zero(alpha) && P##_is_one(beta))) return 0;          \
    for (i = 0; i < n; ++i) {                                                  \
        T *yi = &y[vpos(n, incy, i)];                                          \
        T r = P##_is_zero(beta) ? P##_zero() : P##_mul(beta, *yi);             \
        if (!P##_is_zero(alpha)) {                                             \
            T sum = Pp[i];                                                     \
            for (g = 1; g < nshards; ++g)                                      \
                sum = P##_add(sum, Pp[(long long)g * ldp + i]);                \
            r = P##_add(r, P##_mul(alpha, sum));                               \
        }                                                                      \
        *yi = r;                                                               \
    }                                                                          \
    return 0;                                                                  \
}

DEFINE_COMBINE(oracle_scombine, float, s)
DEFINE_COMBINE(oracle_dcombine, double, d)
DEFINE_COMBINE(oracle_ccombine, ocplx_f, c)
DEFINE_COMBINE(oracle_zcombine, ocplx_d, z)
DEFINE_COMBINE(oracle_wcombine, odd, w)
