// ZHEMV (complex double, Hermitian) kernels and entry point of libxsymv.
#include "xsymv_host.hpp"

namespace xsymv {
template <> const std::vector<KernelSet<cf64>>& kernel_sets<cf64>()
{
    static const std::vector<KernelSet<cf64>> v = {
        make_set<cf64, 4, 8, 8, true>(),    // NB 32, R 512
        make_set<cf64, 4, 16, 4, true>(),   // NB 64, R 256
        make_set<cf64, 8, 8, 8, true>(),    // NB 64, R 512
        make_set<cf64, 4, 8, 8, false>(),   // cached loads
    };
    return v;
}
}  // namespace xsymv

extern "C" int xhemv_z(char uplo, int n, xcomplex128 alpha, const xcomplex128* A, int lda,
                       const xcomplex128* x, int incx, xcomplex128 beta, xcomplex128* y,
                       int incy, void* stream)
{
    using xsymv::cf64;
    return xsymv::symv_impl<cf64>(uplo, n, cf64{alpha.re, alpha.im}, (const cf64*)A, lda,
                                  (const cf64*)x, incx, cf64{beta.re, beta.im}, (cf64*)y, incy,
                                  (hipStream_t)stream);
}
