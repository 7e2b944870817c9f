// CHEMV (complex float, Hermitian) kernels and entry point of libxsymv.
#include "xsymv_host.hpp"

namespace xsymv {
template <> const std::vector<KernelSet<cf32>>& kernel_sets<cf32>()
{
    static const std::vector<KernelSet<cf32>> v = {
        make_set<cf32, 4, 16, 4, true>(),   // NB 64,  R 512
        make_set<cf32, 4, 8, 8, true>(),    // NB 32,  R 1024
        make_set<cf32, 8, 16, 4, true>(),   // NB 128, R 512
        make_set<cf32, 4, 16, 4, false>(),  // cached loads
    };
    return v;
}
}  // namespace xsymv

extern "C" int xhemv_c(char uplo, int n, xcomplex64 alpha, const xcomplex64* A, int lda,
                       const xcomplex64* x, int incx, xcomplex64 beta, xcomplex64* y, int incy,
                       void* stream)
{
    using xsymv::cf32;
    return xsymv::symv_impl<cf32>(uplo, n, cf32{alpha.re, alpha.im}, (const cf32*)A, lda,
                                  (const cf32*)x, incx, cf32{beta.re, beta.im}, (cf32*)y, incy,
                                  (hipStream_t)stream);
}
