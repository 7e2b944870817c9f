// WSYMV (double-double) kernels and entry point of libxsymv.
#include "xsymv_host.hpp"

namespace xsymv {
template <> const std::vector<KernelSet<ddreal>>& kernel_sets<ddreal>()
{
    static const std::vector<KernelSet<ddreal>> v = {
        make_set<ddreal, 4, 8, 4, true>(),   // NB 32, R 256
        make_set<ddreal, 4, 4, 8, true>(),   // NB 16, R 512
        make_set<ddreal, 8, 8, 4, true>(),   // NB 64, R 256
        make_set<ddreal, 4, 8, 4, false>(),  // cached loads
    };
    return v;
}
}  // namespace xsymv

extern "C" int xsymv_w(char uplo, int n, xdd alpha, const xdd* A, int lda, const xdd* x,
                       int incx, xdd beta, xdd* y, int incy, void* stream)
{
    using xsymv::ddreal;
    return xsymv::symv_impl<ddreal>(uplo, n, ddreal{alpha.hi, alpha.lo}, (const ddreal*)A, lda,
                                    (const ddreal*)x, incx, ddreal{beta.hi, beta.lo},
                                    (ddreal*)y, incy, (hipStream_t)stream);
}
