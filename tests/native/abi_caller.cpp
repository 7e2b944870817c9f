// abi_caller.cpp -- a plain host program that uses libxsymv through its C
// header only (no Python, no torch): device buffers from hipMalloc, a
// non-default stream, and results checked against the CPU oracle's C
// functions.  Integer-valued inputs make every summation order exact, so the
// device results must equal the oracle's value for value.
//
// Built by tests/native/build_abi_caller (hipcc, host code only) and run by
// tests/test_gpu_native_abi.py.  Exit status 0: every check passed.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>

extern "C" {
#include "xsymv.h"
#include "xsymv_oracle.h"
}

#define CHECK_HIP(e)                                                          \
    do {                                                                      \
        hipError_t r_ = (e);                                                  \
        if (r_ != hipSuccess) {                                               \
            std::fprintf(stderr, "HIP error %d at line %d\n", (int)r_, __LINE__); \
            return 2;                                                         \
        }                                                                     \
    } while (0)

namespace {

// integers in [-4, 4] from a 64-bit linear congruential sequence
struct Draw {
    unsigned long long s;
    int next()
    {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        return (int)((s >> 33) % 9) - 4;
    }
};

template <class T>
int to_device(const std::vector<T>& h, T** d)
{
    CHECK_HIP(hipMalloc((void**)d, h.size() * sizeof(T) + 16));
    CHECK_HIP(hipMemcpy(*d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
    return 0;
}

int check_dsymv(char uplo, hipStream_t st)
{
    const int n = 777, lda = 780;
    Draw g{uplo == 'L' ? 1ull : 2ull};
    std::vector<double> A((size_t)lda * n, std::nan("")), x(n), y(n);
    for (int j = 0; j < n; ++j)
        for (int i = (uplo == 'U' ? 0 : j); i < (uplo == 'U' ? j + 1 : n); ++i)
            A[(size_t)j * lda + i] = g.next();
    for (int i = 0; i < n; ++i) x[i] = g.next();
    for (int i = 0; i < n; ++i) y[i] = g.next();
    double *dA, *dx, *dy;
    if (to_device(A, &dA) || to_device(x, &dx) || to_device(y, &dy)) return 2;
    int rc = xsymv_d(uplo, n, 1.5, dA, lda, dx, 1, -0.5, dy, 1, st);
    if (rc != 0) {
        std::fprintf(stderr, "xsymv_d returned %d\n", rc);
        return 1;
    }
    // an argument error comes back before any device work
    if (xsymv_d('Q', n, 1.5, dA, lda, dx, 1, -0.5, dy, 1, st) != -1) return 1;
    std::vector<double> got(n);
    CHECK_HIP(hipStreamSynchronize(st));
    CHECK_HIP(hipMemcpy(got.data(), dy, n * sizeof(double), hipMemcpyDeviceToHost));
    std::vector<double> ref = y;
    if (oracle_dsymv(uplo, n, 1.5, A.data(), lda, x.data(), 1, -0.5, ref.data(), 1) != 0) return 2;
    for (int i = 0; i < n; ++i)
        if (got[i] != ref[i]) {
            std::fprintf(stderr, "DSYMV %c row %d: %.17g != %.17g\n", uplo, i, got[i], ref[i]);
            return 1;
        }
    CHECK_HIP(hipFree(dA));
    CHECK_HIP(hipFree(dx));
    CHECK_HIP(hipFree(dy));
    std::printf("dsymv %c n=%d: %d rows equal to the oracle\n", uplo, n, n);
    return 0;
}

int check_zhemv(hipStream_t st)
{
    const int n = 513, lda = 513;
    Draw g{3ull};
    std::vector<xcomplex128> A((size_t)lda * n), x(n), y(n);
    for (auto& a : A) a = {std::nan(""), std::nan("")};
    for (int j = 0; j < n; ++j)
        for (int i = j; i < n; ++i)
            A[(size_t)j * lda + i] = {(double)g.next(), i == j ? 1e3 : (double)g.next()};
    for (auto& v : x) v = {(double)g.next(), (double)g.next()};
    for (auto& v : y) v = {(double)g.next(), (double)g.next()};
    xcomplex128 *dA, *dx, *dy;
    if (to_device(A, &dA) || to_device(x, &dx) || to_device(y, &dy)) return 2;
    const xcomplex128 alpha = {1.5, -0.5}, beta = {0.5, 2.0};
    int rc = xhemv_z('L', n, alpha, dA, lda, dx, 1, beta, dy, 1, st);
    if (rc != 0) {
        std::fprintf(stderr, "xhemv_z returned %d\n", rc);
        return 1;
    }
    std::vector<xcomplex128> got(n);
    CHECK_HIP(hipStreamSynchronize(st));
    CHECK_HIP(hipMemcpy(got.data(), dy, n * sizeof(xcomplex128), hipMemcpyDeviceToHost));
    std::vector<ocplx_d> oA(A.size()), ox(n), oy(n);
    for (size_t k = 0; k < A.size(); ++k) oA[k] = {A[k].re, A[k].im};
    for (int i = 0; i < n; ++i) {
        ox[i] = {x[i].re, x[i].im};
        oy[i] = {y[i].re, y[i].im};
    }
    if (oracle_zhemv('L', n, {alpha.re, alpha.im}, oA.data(), lda, ox.data(), 1,
                     {beta.re, beta.im}, oy.data(), 1) != 0)
        return 2;
    for (int i = 0; i < n; ++i)
        if (got[i].re != oy[i].re || got[i].im != oy[i].im) {
            std::fprintf(stderr, "ZHEMV row %d differs\n", i);
            return 1;
        }
    CHECK_HIP(hipFree(dA));
    CHECK_HIP(hipFree(dx));
    CHECK_HIP(hipFree(dy));
    std::printf("zhemv L n=%d: %d rows equal to the oracle\n", n, n);
    return 0;
}

int check_strmv(hipStream_t st)
{
    const int n = 1000, lda = 1001;
    Draw g{4ull};
    std::vector<float> A((size_t)lda * n, std::nanf("")), x(n);
    for (int j = 0; j < n; ++j)
        for (int i = 0; i <= j; ++i) A[(size_t)j * lda + i] = (float)g.next();
    for (auto& v : x) v = (float)g.next();
    float *dA, *dx;
    if (to_device(A, &dA) || to_device(x, &dx)) return 2;
    int rc = xtrmv_s('U', 'T', 'N', n, dA, lda, dx, 1, st);
    if (rc != 0) {
        std::fprintf(stderr, "xtrmv_s returned %d\n", rc);
        return 1;
    }
    std::vector<float> got(n), ref = x;
    CHECK_HIP(hipStreamSynchronize(st));
    CHECK_HIP(hipMemcpy(got.data(), dx, n * sizeof(float), hipMemcpyDeviceToHost));
    if (oracle_strmv('U', 'T', 'N', n, A.data(), lda, ref.data(), 1) != 0) return 2;
    for (int i = 0; i < n; ++i)
        if (got[i] != ref[i]) {
            std::fprintf(stderr, "STRMV row %d: %g != %g\n", i, got[i], ref[i]);
            return 1;
        }
    CHECK_HIP(hipFree(dA));
    CHECK_HIP(hipFree(dx));
    std::printf("strmv U T n=%d: %d outputs equal to the oracle\n", n, n);
    return 0;
}

}  // namespace

int main()
{
    std::printf("%s\n", xsymv_version());
    hipStream_t st;
    CHECK_HIP(hipStreamCreate(&st));
    int rc = check_dsymv('L', st);
    if (!rc) rc = check_dsymv('U', st);
    if (!rc) rc = check_zhemv(st);
    if (!rc) rc = check_strmv(st);
    if (!rc && xsymv_release() != 0) rc = 1;
    CHECK_HIP(hipStreamDestroy(st));
    std::printf(rc ? "FAILED\n" : "ok\n");
    return rc;
}
