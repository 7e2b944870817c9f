/*
 * xsymv.h -- C ABI of the MI355X (gfx950) symmetric / Hermitian matrix-vector
 * product library (libxsymv.so).
 *
 *   y := alpha*S*x + beta*y
 *
 * S is an n x n symmetric matrix (xsymv_s, xsymv_d, xsymv_w) or Hermitian
 * matrix (xhemv_c, xhemv_z) of which only one triangle is stored and read.
 * The operation is eq.(1) of the CUDA-xSYMV report (Imamura, Mukunoki,
 * Yamada, Machida; IPSJ SIG Technical Report 2014-HPC-146 No.14, §1), and the
 * argument list is the BLAS one the report gives for its API (§2.2 Fig. 5),
 * with the HIP stream appended.  Element types: §2.2 (interleaved complex
 * pairs for [CZ]HEMV, double-double pairs for WSYMV).
 *
 * Arguments (all calls):
 *   uplo   'U'/'u': the upper triangle of A is stored; 'L'/'l': the lower.
 *          The other strict triangle is never read (it may hold anything).
 *   n      order of S, n >= 0.
 *   alpha, beta  host scalars, by value.
 *   A      DEVICE pointer, column-major, element (i, j) at A[i + j*lda];
 *          read only.  For the Hermitian calls the imaginary word of a
 *          diagonal element is never read (it is taken as zero).
 *   lda    leading dimension, lda >= max(1, n).
 *   x      DEVICE pointer, n elements with stride incx (incx != 0; a
 *          negative stride walks the vector backwards, as in BLAS); read only.
 *   y      DEVICE pointer, n elements with stride incy (incy != 0); updated
 *          in place.  With beta == 0 the old y is not read (may hold NaN).
 *   stream a hipStream_t (NULL = the default stream).
 *
 * Ownership: A, x and y belong to the caller and must stay valid until the
 * work enqueued on `stream` has finished.  The library keeps a device
 * workspace per (device, stream), allocated on first use and grown as needed
 * (hipMalloc), never exposed in results, unless the caller installs one with
 * xsymv_set_workspace.  Calls on one stream are ordered; calls on different
 * streams use different workspaces.
 *
 * Behaviour: every call is asynchronous on `stream` (it enqueues kernels and
 * returns).  Results are bitwise identical from run to run for the same
 * inputs, n, uplo and tile configuration: no floating-point atomics are used
 * and partial sums are combined in a fixed order.  n == 0, or alpha == 0 with
 * beta == 1, returns without touching y.  alpha == 0 scales y by beta only
 * (A and x are not read).
 *
 * HIP graphs: the first call of a shape (precision, uplo, n, configuration)
 * builds its work split and uploads it with a synchronising copy, and the
 * first call on a stream may allocate that stream's workspace; neither is
 * allowed while a stream is being captured.  A later call of the same shape
 * on a stream that has already run one enqueues only kernels and can be
 * recorded into a graph and replayed (with timing off).
 *
 * Return codes (checked before any device work; numbering follows the
 * argument positions, as BLAS xerbla does):
 *    0  success
 *   -1  uplo is not one of U, u, L, l
 *   -2  n < 0
 *   -4  A is NULL and n > 0
 *   -5  lda < max(1, n)
 *   -6  x is NULL and n > 0
 *   -7  incx == 0
 *   -9  y is NULL and n > 0
 *  -10  incy == 0
 *  1000 + e  the HIP runtime returned error e (hipError_t) on allocation,
 *            copy or launch.
 *  2000      the workspace the caller installed for this stream
 *            (xsymv_set_workspace) is smaller than the call needs; nothing
 *            was enqueued.
 */
#ifndef XSYMV_H
#define XSYMV_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct { float re, im; } xcomplex64;   /* layout of float2 */
typedef struct { double re, im; } xcomplex128; /* layout of double2 */
typedef struct { double hi, lo; } xdd;         /* value = hi + lo */

/* Precision codes for the helper calls below. */
enum { XSYMV_S = 0, XSYMV_D = 1, XSYMV_C = 2, XSYMV_Z = 3, XSYMV_W = 4 };

/* SSYMV, DSYMV: real symmetric, float / double (report §2.2 Fig. 5). */
int xsymv_s(char uplo, int n, float alpha, const float *A, int lda,
            const float *x, int incx, float beta, float *y, int incy,
            void *stream);
int xsymv_d(char uplo, int n, double alpha, const double *A, int lda,
            const double *x, int incx, double beta, double *y, int incy,
            void *stream);

/* CHEMV, ZHEMV: complex Hermitian (report §2.2 Fig. 5).  The mirrored
 * element is the conjugate: S(j,i) = conj(A(i,j)). */
int xhemv_c(char uplo, int n, xcomplex64 alpha, const xcomplex64 *A, int lda,
            const xcomplex64 *x, int incx, xcomplex64 beta, xcomplex64 *y,
            int incy, void *stream);
int xhemv_z(char uplo, int n, xcomplex128 alpha, const xcomplex128 *A, int lda,
            const xcomplex128 *x, int incx, xcomplex128 beta, xcomplex128 *y,
            int incy, void *stream);

/* WSYMV: double-double symmetric (report §2.2 Fig. 4 and Fig. 5).  Inputs
 * need not be normalised; outputs are (hi, lo) with hi = RN(hi + lo).  The
 * accumulations use double-double multiply-adds with one TwoSum of the high
 * words (the cheaper addition of the double-double library the report
 * builds on), merges and reductions the accurate addition; every result is
 * within 4*n*2^-104*(|alpha|*(|S||x|)_i + |beta|*|y_i|) of the exact value. */
int xsymv_w(char uplo, int n, xdd alpha, const xdd *A, int lda,
            const xdd *x, int incx, xdd beta, xdd *y, int incy,
            void *stream);

/* xGEMV, the general product the report sets SYMV against (a general matrix
 * is read whole and each element used once; the symmetric product reads one
 * triangle and uses each element twice, so it moves half the bytes -- report
 * §1, §2.1):
 *
 *   y := alpha*op(A)*x + beta*y,  op(A) = A (trans 'N'/'n'), A^T ('T'/'t')
 *                                or A^H ('C'/'c'; the same as 'T' for the
 *                                real and double-double types)
 *
 * BLAS xGEMV arguments: A is m x n, column-major, DEVICE pointer, element
 * (i, j) at A[i + j*lda], rows m..lda-1 never read; x has n elements for 'N'
 * and m otherwise, y the other length (DEVICE pointers, strides incx/incy as
 * for the symmetric calls).  Same ownership, asynchrony, determinism,
 * workspace (per device and stream, or installed with xsymv_set_workspace)
 * and beta == 0 / alpha == 0 rules as the symmetric calls.  m == 0, n == 0,
 * or alpha == 0 with beta == 1 return without touching y.
 *
 * Return codes (BLAS xerbla positions, checked before any device work):
 *   -1 trans not N/T/C (either case), -2 m < 0, -3 n < 0, -5 A NULL with
 *   m, n > 0, -6 lda < max(1, m), -7 x NULL, -8 incx == 0, -10 y NULL,
 *   -11 incy == 0; 1000 + hipError_t; 2000 installed workspace too small. */
int xgemv_s(char trans, int m, int n, float alpha, const float *A, int lda,
            const float *x, int incx, float beta, float *y, int incy, void *stream);
int xgemv_d(char trans, int m, int n, double alpha, const double *A, int lda,
            const double *x, int incx, double beta, double *y, int incy, void *stream);
int xgemv_c(char trans, int m, int n, xcomplex64 alpha, const xcomplex64 *A, int lda,
            const xcomplex64 *x, int incx, xcomplex64 beta, xcomplex64 *y, int incy,
            void *stream);
int xgemv_z(char trans, int m, int n, xcomplex128 alpha, const xcomplex128 *A, int lda,
            const xcomplex128 *x, int incx, xcomplex128 beta, xcomplex128 *y, int incy,
            void *stream);
int xgemv_w(char trans, int m, int n, xdd alpha, const xdd *A, int lda, const xdd *x,
            int incx, xdd beta, xdd *y, int incy, void *stream);

/* xGEMV configurations: each precision has a compiled list; info gives
 * waves per workgroup, stripes per wave, columns per group, non-temporal
 * loads (0/1) and rows per strip (outputs may be NULL; returns 0 or -1 for
 * a bad index).  Built in: one configuration per (precision, 'N' or a
 * transposition, size class of m*n: below 12288^2, below 20000^2, larger),
 * the fastest measured on MI355X at one order in each class.  select forces
 * entry idx for every later call of that precision; idx = -1 restores the
 * built-in choice (0 or -1 for a bad code or index).  current: the
 * configuration a call (prec, trans, m, n) runs (-1 for a bad code, trans,
 * m or n).  workspace_bytes: device workspace of one call on the current
 * device with that configuration (-1 cast to size_t on a bad code or when
 * the device cannot be queried).  xgemv_plan: the work split for m x n, strips of R
 * rows and G workgroups (host computation; blocks4 as for xsymv_strip_plan,
 * seg_base[NS+1]); returns the number of workgroups, -1 or -2. */
int xgemv_num_configs(int prec);
int xgemv_config_info(int prec, int idx, int *waves, int *stripes_per_wave,
                      int *cols_per_group, int *nontemporal, int *rows_per_strip);
int xgemv_select_config(int prec, int idx);
int xgemv_current_config(int prec, char trans, int m, int n);
size_t xgemv_workspace_bytes(int prec, char trans, int m, int n);
int xgemv_plan(int m, int n, int R, int G, int *blocks4, int max_blocks, int *seg_base,
               int max_strips);

/* Symmetric / Hermitian rank-2 update on the stored triangle (the report's
 * §5 carries the approach to other Level-2 BLAS; this is SYMV's partner in
 * reductions to tridiagonal form), BLAS xSYR2 / xHER2:
 *
 *   xsyr2_s/d/w:  A := alpha*x*y^T + alpha*y*x^T + A
 *   xher2_c/z:    A := alpha*x*y^H + conj(alpha)*y*x^H + A  (the diagonal
 *                 stays real: its imaginary word is written as zero)
 *
 * uplo as for the symmetric product; only the stored triangle of A (DEVICE
 * pointer, column-major, lda >= max(1, n)) is read and written -- the other
 * triangle and rows n..lda-1 are never touched.  x, y: DEVICE pointers, n
 * elements with strides incx, incy (!= 0; negative walks backwards).
 * Every stored element is updated by one lane in the BLAS reference order
 * (per column j: t1 = alpha*conj(y_j), t2 = conj(alpha*x_j),
 * a := (a + x_i*t1) + y_i*t2; Hermitian diagonal: Re(a) + Re(x_j*t1 +
 * y_j*t2)), without fused multiply-adds, so the results do not depend on the
 * work split.  n == 0 or alpha == 0: nothing is done.  Asynchronous on
 * `stream`; a workspace (2n elements) is used only for non-unit strides.
 * Return codes (BLAS xerbla positions): -1 uplo, -2 n < 0, -4 x NULL,
 * -5 incx == 0, -6 y NULL, -7 incy == 0, -8 A NULL, -9 lda < max(1, n);
 * 1000 + hipError_t; 2000 installed workspace too small. */
int xsyr2_s(char uplo, int n, float alpha, const float *x, int incx, const float *y,
            int incy, float *A, int lda, void *stream);
int xsyr2_d(char uplo, int n, double alpha, const double *x, int incx, const double *y,
            int incy, double *A, int lda, void *stream);
int xher2_c(char uplo, int n, xcomplex64 alpha, const xcomplex64 *x, int incx,
            const xcomplex64 *y, int incy, xcomplex64 *A, int lda, void *stream);
int xher2_z(char uplo, int n, xcomplex128 alpha, const xcomplex128 *x, int incx,
            const xcomplex128 *y, int incy, xcomplex128 *A, int lda, void *stream);
int xsyr2_w(char uplo, int n, xdd alpha, const xdd *x, int incx, const xdd *y, int incy,
            xdd *A, int lda, void *stream);

/* Rank-2 update configurations: waves per workgroup, stripes per wave,
 * columns per group, non-temporal access (0/1), work split (the cost models
 * of xsymv_strip_plan: 0 strip height, doubled in the diagonal triangle; 1
 * stored rows plus strip height; 2 strip height alone) and rows per strip.
 * Built in: one configuration per (precision, triangle, size class of n:
 * below 12288, below 20000, larger), the fastest measured on MI355X at one
 * order in each class.  select forces entry idx for every later call of
 * that precision; idx = -1 restores the built-in choice (0 or -1 for a bad
 * code or index).  current: the configuration a call (prec, uplo, n) runs
 * (-1 for a bad code, uplo or n). */
int xsyr2_num_configs(int prec);
int xsyr2_config_info(int prec, int idx, int *waves, int *stripes_per_wave,
                      int *cols_per_group, int *nontemporal, int *split,
                      int *rows_per_strip);
int xsyr2_select_config(int prec, int idx);
int xsyr2_current_config(int prec, char uplo, int n);

/* One GPU's share of the product, for the path sharded over several GPUs
 * (the report's §5 points to multi-GPU SYMV, its ref. [7]); on one GPU the
 * shards run one after another.  The columns are cut into panels of `panel`
 * consecutive columns (the last may be short), dealt to `nshards` shards
 * round by round: in even rounds shard g takes the round's g-th panel, in
 * odd rounds its (nshards-1-g)-th, which keeps the shards' triangle areas
 * close.  xsymv_shard_columns writes the global columns of `shard`
 * (ascending; cols may be NULL) and returns their count (-1: bad argument);
 * a host computation.
 *
 *   x[sd]symv_shard_X / xhemv_shard_[cz]:  p := the shard's share of S*x --
 *   every stored element A(i,j) of an owned column j taken in both roles
 *   (p_i += A(i,j) x_j, and p_j += conj(A(i,j)) x_i for i != j), the
 *   diagonal once (Hermitian: its real word) -- so that the shards' partials
 *   add up to S*x.
 *
 * Aloc: DEVICE pointer to the shard's local matrix, its columns in ascending
 * global order, each a full column of A (rows 0..n-1 at stride lda >=
 * max(1, n); only the uplo triangle is read).  x: DEVICE, n elements, stride
 * incx != 0.  p: DEVICE, n contiguous elements, overwritten (zeros when the
 * shard owns no column).  Deterministic: fixed-order partial sums, no
 * atomics.  Asynchronous on `stream`; uses the per-stream workspace
 * (xsymv_shard_workspace_bytes).  Codes: -1 uplo, -2 n < 0, -3 panel <= 0,
 * -4 nshards <= 0, -5 shard outside [0, nshards), -6 Aloc NULL while the
 * shard owns columns, -7 lda < max(1, n), -8 x NULL, -9 incx == 0,
 * -10 p NULL; 1000 + hipError_t; 2000 installed workspace too small.
 *
 *   xsymv_combine_X / xhemv_combine_[cz]:  y := beta*y + alpha*(P[0] + P[1]
 *   + ... + P[nshards-1]), partial g at P + g*ldp (DEVICE, n elements each),
 *   summed in rank order -- the fixed order that keeps the result the same
 *   from run to run, whatever the exchange did.  BLAS rules: beta == 0 does
 *   not read y, alpha == 0 does not read P, n == 0 or (alpha == 0 and
 *   beta == 1) returns at once.  y: DEVICE, stride incy != 0.  Codes: -1 n,
 *   -2 nshards <= 0, -4 P NULL, -5 ldp < max(1, n), -7 y NULL, -8 incy == 0;
 *   1000 + hipError_t. */
int xsymv_shard_columns(int n, int panel, int nshards, int shard, int *cols);
/* The work split of one shard's product (host computation, as
 * xsymv_strip_plan, over the shard's local columns): blocks4, strip_base and
 * seg_base as there, col0 (NS entries) the first local column of each
 * strip's sequence.  A strip without any of the shard's columns has an empty
 * sequence and (unless a workgroup's range steps through it) no segment.
 * Returns the number of workgroups (0 when the shard owns no column), -1 for
 * bad arguments, -2 if an output is too small. */
int xsymv_shard_plan(char uplo, int n, int R, int G, int split, int panel, int nshards,
                     int shard, int *blocks4, int max_blocks, int *strip_base, int *seg_base,
                     int *col0, int max_strips);
size_t xsymv_shard_workspace_bytes(int prec, char uplo, int n, int panel, int nshards,
                                   int shard);
int xsymv_shard_s(char uplo, int n, int panel, int nshards, int shard, const float *Aloc,
                  int lda, const float *x, int incx, float *p, void *stream);
int xsymv_shard_d(char uplo, int n, int panel, int nshards, int shard, const double *Aloc,
                  int lda, const double *x, int incx, double *p, void *stream);
int xhemv_shard_c(char uplo, int n, int panel, int nshards, int shard,
                  const xcomplex64 *Aloc, int lda, const xcomplex64 *x, int incx,
                  xcomplex64 *p, void *stream);
int xhemv_shard_z(char uplo, int n, int panel, int nshards, int shard,
                  const xcomplex128 *Aloc, int lda, const xcomplex128 *x, int incx,
                  xcomplex128 *p, void *stream);
int xsymv_shard_w(char uplo, int n, int panel, int nshards, int shard, const xdd *Aloc,
                  int lda, const xdd *x, int incx, xdd *p, void *stream);
int xsymv_combine_s(int n, int nshards, float alpha, const float *P, int ldp, float beta,
                    float *y, int incy, void *stream);
int xsymv_combine_d(int n, int nshards, double alpha, const double *P, int ldp, double beta,
                    double *y, int incy, void *stream);
int xhemv_combine_c(int n, int nshards, xcomplex64 alpha, const xcomplex64 *P, int ldp,
                    xcomplex64 beta, xcomplex64 *y, int incy, void *stream);
int xhemv_combine_z(int n, int nshards, xcomplex128 alpha, const xcomplex128 *P, int ldp,
                    xcomplex128 beta, xcomplex128 *y, int incy, void *stream);
int xsymv_combine_w(int n, int nshards, xdd alpha, const xdd *P, int ldp, xdd beta, xdd *y,
                    int incy, void *stream);

/* Triangular matrix-vector product (another of the Level-2 BLAS the report's
 * §5 carries the approach to), BLAS xTRMV:
 *
 *   x := op(T)*x,   op(T) = T ('N'), T^T ('T') or T^H ('C'; = 'T' for the
 *                   real types s, d, w)
 *
 * T is the uplo triangle of A (DEVICE pointer, column-major, lda >=
 * max(1, n)); diag 'N' takes the diagonal from A, 'U' takes ones and never
 * reads it.  The other triangle and rows n..lda-1 are never read.  x: DEVICE
 * pointer, n elements with stride incx (!= 0; negative walks backwards),
 * overwritten in place; gaps between strided elements are left alone.  Each
 * output is a fixed-order sum of partial sums (no atomics), so repeated calls
 * give identical bits.  The library reads all of x before it writes any of
 * it.  n == 0: nothing is done.  Asynchronous on `stream`; uses the
 * per-stream workspace (xtrmv_workspace_bytes).  Return codes (BLAS xerbla
 * positions): -1 uplo, -2 trans, -3 diag, -4 n < 0, -5 A NULL,
 * -6 lda < max(1, n), -7 x NULL, -8 incx == 0; 1000 + hipError_t; 2000
 * installed workspace too small. */
int xtrmv_s(char uplo, char trans, char diag, int n, const float *A, int lda, float *x,
            int incx, void *stream);
int xtrmv_d(char uplo, char trans, char diag, int n, const double *A, int lda, double *x,
            int incx, void *stream);
int xtrmv_c(char uplo, char trans, char diag, int n, const xcomplex64 *A, int lda,
            xcomplex64 *x, int incx, void *stream);
int xtrmv_z(char uplo, char trans, char diag, int n, const xcomplex128 *A, int lda,
            xcomplex128 *x, int incx, void *stream);
int xtrmv_w(char uplo, char trans, char diag, int n, const xdd *A, int lda, xdd *x,
            int incx, void *stream);

/* Triangular product configurations, same fields as the rank-2 update's.
 * Built in: one configuration per (precision, triangle, 'N' or a
 * transposition, size class of n: below 12288, below 20000, larger), the
 * fastest measured on MI355X at one order in each class.
 * xtrmv_select_config(prec, idx) forces configuration idx for every call of
 * that precision; idx = -1 restores the built-in choice (0, or -1 for a bad
 * code or index).  xtrmv_current_config: the configuration a call (prec,
 * uplo, trans, n) would use now (-1 for a bad code, uplo, trans or n).  xtrmv_workspace_bytes:
 * device workspace bytes of one call (precision, uplo, trans, n) with that
 * configuration on the current device (0 for n <= 0; -1 cast to size_t on a
 * bad precision code or when the device cannot be queried). */
int xtrmv_num_configs(int prec);
int xtrmv_config_info(int prec, int idx, int *waves, int *stripes_per_wave,
                      int *cols_per_group, int *nontemporal, int *split,
                      int *rows_per_strip);
int xtrmv_select_config(int prec, int idx);
int xtrmv_current_config(int prec, char uplo, char trans, int n);
size_t xtrmv_workspace_bytes(int prec, char uplo, char trans, int n);

/* Bytes of device workspace one call of precision `prec` and order n uses
 * with the configuration selected for it now, on the current device (0 for
 * n == 0; -1 cast to size_t for a bad precision code, or when the device
 * cannot be queried: the row-strip family's split depends on how many of
 * its workgroups the device holds at once). */
size_t xsymv_workspace_bytes(int prec, char uplo, int n);

/* Install a caller-owned device buffer of `bytes` bytes as the workspace of
 * `stream` on the current device (the optional caller-owned workspace of the
 * boundary; size it with xsymv_workspace_bytes).  Calls on that stream then
 * use it and never allocate a workspace; a call that needs more than `bytes`
 * returns 2000.  The buffer must stay valid, and must not be used by anything
 * else, while calls on the stream may still run; the library never frees it.
 * dev_ptr = NULL (with bytes = 0) removes an installed buffer, so the
 * library owns the stream's workspace again.  Replacing or removing waits for
 * the work queued on `stream` and frees a library-owned buffer of it.
 * Returns 0, -2 (NULL with bytes > 0) or 1000 + hipError_t.  Cached plans
 * (a few KB per order and configuration) are still allocated by the library. */
int xsymv_set_workspace(void *dev_ptr, size_t bytes, void *stream);

/* SSYMV for callers that cannot allocate device memory -- code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same product, arguments, return codes, configuration choice, kernels and
 * work split as xsymv_s, hence the same bytes; but no device memory is ever
 * allocated (no hipMalloc, hipFree or pinned host memory, and no timing
 * events: xsymv_timing_* does not see these calls).  The partial sums and the
 * work split live in one static device array of XSYMV_STATIC_SCRATCH_BYTES
 * per GPU, part of the library's code object (every GPU the library runs on
 * holds it until the process ends).
 *
 * The first call of a shape (uplo, n, configuration) on a GPU writes the work
 * split into the array with a copy from host memory and waits for `stream`
 * (so it cannot be captured); later calls of that shape enqueue kernels only.
 * Calls on one GPU share the array: calls on one stream are ordered, but calls
 * that overlap in time on one GPU (other streams, other threads) race on it
 * and must not be issued.  Extra return codes, checked before any device work:
 *   3000  the call needs more than XSYMV_STATIC_SCRATCH_BYTES (partials of
 *         the configuration chosen for n, plus x gathered when incx != 1);
 *   3001  the configuration selected for (uplo, n) by a caller rule is not a
 *         row-strip one (column_runs 4, 5 or 6) -- only those are supported;
 *   3002  the current device index is 64 or more. */
#define XSYMV_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
int xsymv_s_noalloc(char uplo, int n, float alpha, const float *A, int lda,
                    const float *x, int incx, float beta, float *y, int incy,
                    void *stream);

/* Release every library-owned workspace and cached tile plan of the current
 * device and forget installed workspaces (synchronises the device first).
 * Returns 0 or 1000 + hipError_t. */
int xsymv_release(void);

/* Tile configurations (the autotuner's search space, report §3 Table 1
 * plays this role for the report's CUDA kernels).  Each precision has a
 * fixed list of compiled configurations; xsymv_config_info describes entry
 * `idx`: waves per workgroup, columns per wave (row-strip family: columns
 * per group), stripes per tile (row-strip: waves x stripes per wave), rows
 * per stripe, non-temporal loads of A (0/1), x rows staged in LDS (0/1), and
 * the kernel family: 0 tiles, whole tile unrolled; 1 tiles, each wave walks
 * its columns one contiguous run at a time; 2 the same with the next run
 * prefetched; 3 tiles, all waves of a workgroup on one column; 4 row strips,
 * work split by strip height, doubled in the diagonal triangle; 5 row strips,
 * work split by stored rows plus strip height; 6 row strips, work split by
 * strip height alone.  Any output pointer may be NULL.  Returns 0, or -1 for a bad
 * index. */
int xsymv_num_configs(int prec);
int xsymv_config_info(int prec, int idx, int *waves, int *cols_per_wave,
                      int *stripes, int *rows_per_stripe, int *nontemporal,
                      int *x_in_lds, int *column_runs);

/* Select the configuration used for precision `prec`, uplo and every n in
 * [n_lo, n_hi] (later selections take precedence).  idx = -1 restores the
 * built-in choice for that range.  Returns 0 or -1 for bad arguments.
 *
 * Built-in choice: per (precision, uplo, range of n, stride class of lda),
 * the configuration the on-device autotuner measured fastest on MI355X over
 * a grid of orders from 64 to 32768 (the counterpart of the report's
 * per-size rules, §3 Table 3).  Stride class 0: lda * element size is a
 * multiple of 64 bytes (measured with lda = n); class 1: any other lda
 * (measured with lda = n + 1; where it has no rule, class 0's applies).
 * Entry 0 where no rule applies.  Caller selections (this call, autotune,
 * load_config) take precedence over it, for every lda. */
int xsymv_select_config(int prec, char uplo, int n_lo, int n_hi, int idx);
/* Configuration index that a call (prec, uplo, n) with a class-0 leading
 * dimension would use now; the _lda form for a given lda (-1 for a bad
 * precision or lda < 1). */
int xsymv_current_config(int prec, char uplo, int n);
int xsymv_current_config_lda(int prec, char uplo, int n, int lda);

/* Autotuner (the report's §3 tunes its CUDA kernels offline per GPU; this
 * is the on-device counterpart).  On the current device and `stream`, time
 * every compiled configuration of `prec` for (uplo, n) on device-generated
 * data: two warm-up calls, then `reps` timed calls each (HIP events; caches
 * flushed before each call when the matrix is under 1 GiB).  The lowest
 * median wins (ties: the lower index) and is installed for every n in
 * [n_lo, n_hi], as xsymv_select_config does.  Allocates, uses and frees
 * n*n elements of matrix plus vectors (and a 1 GiB flush buffer for small
 * matrices); synchronises `stream`.  best_idx and ms (median per
 * configuration, at most max_cfg entries) may be NULL.  Returns 0, -1 for a
 * bad argument, or 1000 + hipError_t. */
int xsymv_autotune(int prec, char uplo, int n, int n_lo, int n_hi, int reps,
                   void *stream, int *best_idx, float *ms, int max_cfg);
/* The same search on a matrix of leading dimension lda (>= n; -1 otherwise):
 * xsymv_autotune is this call with lda = n.  The installed rule applies to
 * every leading dimension. */
int xsymv_autotune_lda(int prec, char uplo, int n, int lda, int n_lo, int n_hi,
                       int reps, void *stream, int *best_idx, float *ms, int max_cfg);

/* Selection rules as a JSON file: {"library": ..., "rules": [{"prec": "s",
 * "uplo": "L", "n_lo": .., "n_hi": .., "waves": .., "cols_per_wave": ..,
 * "stripes": .., "nontemporal": .., "x_in_lds": .., "column_runs": ..},
 * ...]}.  Rules are matched to compiled
 * configurations by shape.  save: 0 or -1 (cannot write).  load: number of
 * rules installed (appended after the current ones, so they take
 * precedence), -1 (cannot read) or -2 (malformed).  clear: drop every caller
 * rule (back to the built-in choice).  save writes the caller rules only. */
int xsymv_save_config(const char *path);
int xsymv_load_config(const char *path);
int xsymv_clear_config(void);

/* Kernel timing for measurement.  xsymv_timing_enable(mode): 0 off (the
 * default); 1 every call times its main (streaming) kernel and its merge
 * kernel; 2 every call times itself whole.  The HIP events are bound to the
 * launches (hipExtLaunchKernel's start and stop events), so they take the
 * kernels' own start and end times.  Mode 1: main_ms runs from the main
 * kernel's start to its end, merge_ms from there to the merge's end (the
 * launch gap included).  Mode 2: no event is bound between the two kernels
 * (binding one there delays the merge by a few microseconds); main_ms is the
 * call's span, from the main kernel's start to the merge's end, and merge_ms
 * is 0.  Calls of one kernel (the rank-2 update, the shard combination)
 * record that kernel as main_ms and 0 in either mode.  xsymv_timing_read
 * waits for the recorded events, writes up to `max` (main_ms, merge_ms)
 * pairs, clears the record and returns how many it wrote (or
 * 1000 + hipError_t on failure).  xsymv_timing_enable returns 0, or -1 for
 * a mode other than 0, 1, 2. */
int xsymv_timing_enable(int mode);
int xsymv_timing_read(float *main_ms, float *merge_ms, int max);

/* Workgroups a row-strip configuration (column_runs 4, 5 or 6) is launched with
 * on the current device: the number of its workgroups the device holds at
 * once.  0 for other families, -1 for a bad index, -(1000 + hipError_t) on a
 * runtime error. */
int xsymv_config_workgroups(int prec, int idx, char uplo);

/* The row-strip work split the library uses for order n, strips of R rows,
 * G workgroups and cost model `split` (0: every column of a strip costs the
 * strip's height, doubled in its diagonal triangle -- family 4; 1: a column
 * costs its stored rows plus the strip's height -- family 5; 2: every column
 * costs the strip's height -- family 6), a host
 * computation with no device work: writes per workgroup
 * {first, end} of its range in the strips' concatenated column sequence,
 * its first segment slot and the strip of `first` into blocks4 (4 ints per
 * workgroup), the sequence position where each strip starts (NS+1 entries)
 * into strip_base and each strip's first segment slot (NS+1 entries, the
 * last = total segments) into seg_base.  Returns the number of workgroups
 * used, -1 for bad arguments, -2 if an output is too small. */
int xsymv_strip_plan(char uplo, int n, int R, int G, int split, int *blocks4,
                     int max_blocks, int *strip_base, int *seg_base, int max_strips);

/* Measurement helper: the device's plain streaming-read bandwidth, the
 * reference for "% of a measured stream-read peak" (the report puts its
 * results against both the specification and a measured bandwidth, §4).
 * Allocates `bytes` (>= 64 MiB) of device memory, fills it, then, for each
 * of ten layouts, times `reps` launches (after one warm-up) on `stream`:
 * 2048, 8192 or 32768 workgroups of 256 lanes, each reading its own
 * contiguous chunk with 4 or 8 non-temporal 16-byte loads in flight per
 * lane; and 256 or 512 workgroups of 1024 lanes sweeping the buffer together
 * in tiles of 2 or 4 such loads per lane (tile t to workgroup t mod grid).
 * Frees the buffer and synchronises the stream.  Writes the best layout's
 * median rate and the best single launch in GB/s (either may be NULL).
 * Returns 0, -1 for bad arguments or 1000 + hipError_t. */
int xsymv_read_bandwidth(size_t bytes, int reps, void *stream, float *gbps,
                         float *best_gbps);

/* Measurement helper: the device's plain read + write bandwidth, the
 * reference for the rank-2 update, which reads the stored triangle and
 * writes it back (the report sets its results beside a measured copy rate as
 * well as the specification, §4).  Allocates 2 * `bytes` (bytes >= 64 MiB),
 * fills them, then for each of four layouts (2048 or 8192 workgroups of 256
 * lanes, each copying its own contiguous chunk from one buffer to the other
 * with 4 or 8 non-temporal 16-byte loads and stores in flight per lane) times
 * `reps` launches after one warm-up.  Rates count the bytes read plus the
 * bytes written.  Writes the best layout's median rate and the best single
 * launch in GB/s (either may be NULL); frees the buffer and synchronises the
 * stream.  Returns 0, -1 for bad arguments or 1000 + hipError_t. */
int xsymv_copy_bandwidth(size_t bytes, int reps, void *stream, float *gbps, float *best_gbps);

/* Library version string. */
const char *xsymv_version(void);

#ifdef __cplusplus
}
#endif
#endif
