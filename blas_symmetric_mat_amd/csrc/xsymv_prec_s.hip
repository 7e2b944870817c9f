// SSYMV (float) kernels and entry point of libxsymv.
#include "xsymv_host.hpp"

namespace xsymv {
template <> const std::vector<KernelSet<float>>& kernel_sets<float>()
{
    static const std::vector<KernelSet<float>> v = {
        make_set<float, 4, 16, 4, true>(),   // NB 64,  R 1024
        make_set<float, 4, 16, 2, true>(),   // NB 64,  R 512
        make_set<float, 4, 32, 2, true>(),   // NB 128, R 512
        make_set<float, 8, 16, 4, true>(),   // NB 128, R 1024
        make_set<float, 4, 16, 4, false>(),  // cached loads
    };
    return v;
}
}  // namespace xsymv

extern "C" int xsymv_s(char uplo, int n, float alpha, const float* A, int lda, const float* x,
                       int incx, float beta, float* y, int incy, void* stream)
{
    return xsymv::symv_impl<float>(uplo, n, alpha, A, lda, x, incx, beta, y, incy,
                                   (hipStream_t)stream);
}
