// DSYMV (double) kernels and entry point of libxsymv.
#include "xsymv_host.hpp"

namespace xsymv {
template <> const std::vector<KernelSet<double>>& kernel_sets<double>()
{
    static const std::vector<KernelSet<double>> v = {
        make_set<double, 4, 16, 4, true>(),   // NB 64,  R 512
        make_set<double, 4, 16, 8, true>(),   // NB 64,  R 1024
        make_set<double, 4, 32, 4, true>(),   // NB 128, R 512
        make_set<double, 8, 16, 4, true>(),   // NB 128, R 512
        make_set<double, 4, 16, 4, false>(),  // cached loads
    };
    return v;
}
}  // namespace xsymv

extern "C" int xsymv_d(char uplo, int n, double alpha, const double* A, int lda,
                       const double* x, int incx, double beta, double* y, int incy,
                       void* stream)
{
    return xsymv::symv_impl<double>(uplo, n, alpha, A, lda, x, incx, beta, y, incy,
                                    (hipStream_t)stream);
}
