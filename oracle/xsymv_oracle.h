/*
 * xsymv_oracle.h -- interface of the CPU oracle for y := alpha*S*x + beta*y.
 *
 * TEST INFRASTRUCTURE ONLY.  The oracle is a plain, slow, sequential C
 * implementation used by the test suite, by the packaged smoke check and by
 * the benchmark's CPU-baseline leg.  No product code path may call it.  It
 * shares no source with the GPU library.
 *
 * Source of the method: Imamura, Mukunoki, Yamada, Machida, "CUDA-xSYMV no
 * jisso to hyoka" (Implementation and evaluation of CUDA-xSYMV), IPSJ SIG
 * Technical Report 2014-HPC-146 No.14 -- cited below as "the CUDA-xSYMV
 * report".  Problem statement: §1 eq.(1), which the product follows as
 * written; BLAS-style argument list: §2.2 Fig. 5; element types
 * (float2 / double2 complex, double2 double-double): §2.2.
 *
 * Matrices are column-major: element (i, j) of A lives at A[i + j*lda],
 * 0-based.  Vectors use BLAS increments: X(k) = x[kx + k*incx] with
 * kx = 0 for incx > 0 and kx = (1-n)*incx for incx < 0.
 *
 * Return codes (same numbering as the product library, BLAS xerbla order):
 *   0 ok, -1 bad uplo, -2 n < 0, -4 A NULL, -5 lda < max(1,n),
 *   -6 x NULL, -7 incx == 0, -9 y NULL, -10 incy == 0.
 */
#ifndef XSYMV_ORACLE_H
#define XSYMV_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

typedef struct { float re, im; } ocplx_f;    /* interleaved, like float2  */
typedef struct { double re, im; } ocplx_d;   /* interleaved, like double2 */
typedef struct { double hi, lo; } odd;       /* value = hi + lo exactly   */

/* Full result from the definition of eq.(1), output by output:
 *   y(i) := beta*y(i) + alpha * sum_{j ascending} S(i,j)*x(j)
 * where S is the full matrix implied by the stored triangle (the mirrored
 * element conjugated for Hermitian matrices, whose diagonal is its real
 * word); BLAS rules for beta == 0 (y not read), alpha == 0 and increments.
 * The outputs are independent: the rows are spread over
 * oracle_set_threads() threads, with the same bits for any count. */
int oracle_ssymv(char uplo, int n, float alpha, const float *A, int lda,
                 const float *x, int incx, float beta, float *y, int incy);
int oracle_dsymv(char uplo, int n, double alpha, const double *A, int lda,
                 const double *x, int incx, double beta, double *y, int incy);
int oracle_chemv(char uplo, int n, ocplx_f alpha, const ocplx_f *A, int lda,
                 const ocplx_f *x, int incx, ocplx_f beta, ocplx_f *y, int incy);
int oracle_zhemv(char uplo, int n, ocplx_d alpha, const ocplx_d *A, int lda,
                 const ocplx_d *x, int incx, ocplx_d beta, ocplx_d *y, int incy);
int oracle_wsymv(char uplo, int n, odd alpha, const odd *A, int lda,
                 const odd *x, int incx, odd beta, odd *y, int incy);

/* Threads of the full-product calls (default 1): 0, -1 for nthreads < 1,
 * -2 when built without OpenMP and nthreads > 1.  get: the current count. */
int oracle_set_threads(int nthreads);
int oracle_get_threads(void);

/* Selected rows only, the same definition of eq.(1):
 *   out[r] = beta*y(rows[r]) + alpha * sum_{j ascending} S(rows[r], j)*x(j)
 * where S is the full matrix implied by the stored triangle.  y is read
 * (not written); results go to out[0..nrows).  Used to check very large
 * problems on a sample of rows.  Same argument checks as above, plus
 * -11 for a row index outside [0, n). */
int oracle_ssymv_rows(char uplo, int n, float alpha, const float *A, int lda,
                      const float *x, int incx, float beta, const float *y,
                      int incy, const long long *rows, int nrows, float *out);
int oracle_dsymv_rows(char uplo, int n, double alpha, const double *A, int lda,
                      const double *x, int incx, double beta, const double *y,
                      int incy, const long long *rows, int nrows, double *out);
int oracle_chemv_rows(char uplo, int n, ocplx_f alpha, const ocplx_f *A, int lda,
                      const ocplx_f *x, int incx, ocplx_f beta, const ocplx_f *y,
                      int incy, const long long *rows, int nrows, ocplx_f *out);
int oracle_zhemv_rows(char uplo, int n, ocplx_d alpha, const ocplx_d *A, int lda,
                      const ocplx_d *x, int incx, ocplx_d beta, const ocplx_d *y,
                      int incy, const long long *rows, int nrows, ocplx_d *out);
int oracle_wsymv_rows(char uplo, int n, odd alpha, const odd *A, int lda,
                      const odd *x, int incx, odd beta, const odd *y,
                      int incy, const long long *rows, int nrows, odd *out);

/* General matrix-vector product, BLAS xGEMV: y := alpha*op(A)*x + beta*y
 * with op(A) = A ('N'), A^T ('T') or A^H ('C'; 'T' for the real and
 * double-double types), A m x n.  x has n elements for 'N' and m otherwise,
 * y the other length.  Every output element from the definition (inner index
 * ascending).  Return codes (BLAS xerbla positions): -1 trans, -2 m < 0,
 * -3 n < 0, -5 A NULL, -6 lda < max(1,m), -7 x NULL, -8 incx == 0,
 * -10 y NULL, -11 incy == 0.  The _rows variants write outputs rows[] to out
 * (y is read, not written; -12 for an index outside y). */
int oracle_sgemv(char trans, int m, int n, float alpha, const float *A, int lda,
                 const float *x, int incx, float beta, float *y, int incy);
int oracle_dgemv(char trans, int m, int n, double alpha, const double *A, int lda,
                 const double *x, int incx, double beta, double *y, int incy);
int oracle_cgemv(char trans, int m, int n, ocplx_f alpha, const ocplx_f *A, int lda,
                 const ocplx_f *x, int incx, ocplx_f beta, ocplx_f *y, int incy);
int oracle_zgemv(char trans, int m, int n, ocplx_d alpha, const ocplx_d *A, int lda,
                 const ocplx_d *x, int incx, ocplx_d beta, ocplx_d *y, int incy);
int oracle_wgemv(char trans, int m, int n, odd alpha, const odd *A, int lda,
                 const odd *x, int incx, odd beta, odd *y, int incy);
int oracle_sgemv_rows(char trans, int m, int n, float alpha, const float *A, int lda,
                      const float *x, int incx, float beta, const float *y, int incy,
                      const long long *rows, int nrows, float *out);
int oracle_dgemv_rows(char trans, int m, int n, double alpha, const double *A, int lda,
                      const double *x, int incx, double beta, const double *y, int incy,
                      const long long *rows, int nrows, double *out);
int oracle_cgemv_rows(char trans, int m, int n, ocplx_f alpha, const ocplx_f *A,
                      int lda, const ocplx_f *x, int incx, ocplx_f beta,
                      const ocplx_f *y, int incy, const long long *rows, int nrows,
                      ocplx_f *out);
int oracle_zgemv_rows(char trans, int m, int n, ocplx_d alpha, const ocplx_d *A,
                      int lda, const ocplx_d *x, int incx, ocplx_d beta,
                      const ocplx_d *y, int incy, const long long *rows, int nrows,
                      ocplx_d *out);
int oracle_wgemv_rows(char trans, int m, int n, odd alpha, const odd *A, int lda,
                      const odd *x, int incx, odd beta, const odd *y, int incy,
                      const long long *rows, int nrows, odd *out);

/* Symmetric / Hermitian rank-2 update on the stored triangle, BLAS xSYR2 /
 * xHER2: A := alpha*x*y^T + alpha*y*x^T + A (real, double-double) or
 * A := alpha*x*y^H + conj(alpha)*y*x^H + A (complex; the diagonal stays real,
 * its imaginary word is set to zero).  BLAS reference order per column j:
 * t1 = alpha*conj(y(j)), t2 = conj(alpha*x(j)), A(i,j) := (A(i,j) +
 * x(i)*t1) + y(i)*t2.  The other triangle is neither read nor written.
 * Return codes: -1 uplo, -2 n < 0, -4 x NULL, -5 incx == 0, -6 y NULL,
 * -7 incy == 0, -8 A NULL, -9 lda < max(1,n).  n == 0 or alpha == 0: no
 * change. */
int oracle_ssyr2(char uplo, int n, float alpha, const float *x, int incx,
                 const float *y, int incy, float *A, int lda);
int oracle_dsyr2(char uplo, int n, double alpha, const double *x, int incx,
                 const double *y, int incy, double *A, int lda);
int oracle_cher2(char uplo, int n, ocplx_f alpha, const ocplx_f *x, int incx,
                 const ocplx_f *y, int incy, ocplx_f *A, int lda);
int oracle_zher2(char uplo, int n, ocplx_d alpha, const ocplx_d *x, int incx,
                 const ocplx_d *y, int incy, ocplx_d *A, int lda);
int oracle_wsyr2(char uplo, int n, odd alpha, const odd *x, int incx,
                 const odd *y, int incy, odd *A, int lda);

/* Triangular matrix-vector product, BLAS xTRMV: x := op(T)*x, T the stored
 * triangle (uplo) of A, diag 'N' (diagonal from A) or 'U' (unit diagonal,
 * not read), trans 'N', 'T' or 'C'.  Every output from the definition (inner
 * index ascending), x overwritten after all outputs are formed.  Return
 * codes: -1 uplo, -2 trans, -3 diag, -4 n < 0, -5 A NULL, -6 lda < max(1,n),
 * -7 x NULL, -8 incx == 0. */
int oracle_strmv(char uplo, char trans, char diag, int n, const float *A, int lda,
                 float *x, int incx);
int oracle_dtrmv(char uplo, char trans, char diag, int n, const double *A, int lda,
                 double *x, int incx);
int oracle_ctrmv(char uplo, char trans, char diag, int n, const ocplx_f *A, int lda,
                 ocplx_f *x, int incx);
int oracle_ztrmv(char uplo, char trans, char diag, int n, const ocplx_d *A, int lda,
                 ocplx_d *x, int incx);
int oracle_wtrmv(char uplo, char trans, char diag, int n, const odd *A, int lda,
                 odd *x, int incx);

/* One shard's partial product and the rank-ordered combination (the path
 * sharded over several GPUs).  Panels of `panel` columns are dealt to
 * `nshards` shards round by round in boustrophedon order; Aloc holds the
 * shard's columns in ascending order (stride lda).  p (n elements,
 * contiguous) := the shard's share of S*x: output i sums, j ascending, the
 * terms S(i,j)*x(j) whose element is stored in an owned column (column j
 * when (i,j) is in the stored triangle, column i otherwise).  Codes: -1 uplo, -2 n,
 * -3 panel <= 0, -4 nshards <= 0, -5 shard out of range, -6 Aloc NULL,
 * -7 lda, -8 x NULL, -9 incx == 0, -10 p NULL.
 * oracle_Xcombine: y := beta*y + alpha*(P[0] + P[1] + ...), partial g at
 * P + g*ldp, summed in ascending g; codes -1 n, -2 nshards, -4 P NULL,
 * -5 ldp, -7 y NULL, -8 incy == 0.
 * oracle_shard_columns: the shard's global columns, ascending (cols may be
 * NULL); returns their count, or -1 for bad arguments. */
int oracle_shard_columns(int n, int panel, int nshards, int shard, int *cols);
int oracle_ssymv_shard(char uplo, int n, int panel, int nshards, int shard, const float *Aloc,
                       int lda, const float *x, int incx, float *p);
int oracle_dsymv_shard(char uplo, int n, int panel, int nshards, int shard, const double *Aloc,
                       int lda, const double *x, int incx, double *p);
int oracle_chemv_shard(char uplo, int n, int panel, int nshards, int shard, const ocplx_f *Aloc,
                       int lda, const ocplx_f *x, int incx, ocplx_f *p);
int oracle_zhemv_shard(char uplo, int n, int panel, int nshards, int shard, const ocplx_d *Aloc,
                       int lda, const ocplx_d *x, int incx, ocplx_d *p);
int oracle_wsymv_shard(char uplo, int n, int panel, int nshards, int shard, const odd *Aloc,
                       int lda, const odd *x, int incx, odd *p);
int oracle_scombine(int n, int nshards, float alpha, const float *P, int ldp, float beta,
                    float *y, int incy);
int oracle_dcombine(int n, int nshards, double alpha, const double *P, int ldp, double beta,
                    double *y, int incy);
int oracle_ccombine(int n, int nshards, ocplx_f alpha, const ocplx_f *P, int ldp, ocplx_f beta,
                    ocplx_f *y, int incy);
int oracle_zcombine(int n, int nshards, ocplx_d alpha, const ocplx_d *P, int ldp, ocplx_d beta,
                    ocplx_d *y, int incy);
int oracle_wcombine(int n, int nshards, odd alpha, const odd *P, int ldp, odd beta, odd *y,
                    int incy);

/* The double-double primitives, exported so that the tests can pin them
 * one by one against exact rational arithmetic. */
odd oracle_dd_add(odd a, odd b);
odd oracle_dd_mul(odd a, odd b);

#ifdef __cplusplus
}
#endif
#endif
