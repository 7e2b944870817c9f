// ZHEMV (complex double, Hermitian) kernels and entry point of libxsymv.
#include "xsymv_host.hpp"

namespace xsymv {
template <> const std::vector<KernelSet<cf64>>& kernel_sets<cf64>()
{
    // index 0 is the built-in default (fastest streaming kernel measured on MI355X
    // at the largest benchmark size of this precision)
    static const std::vector<KernelSet<cf64>> v = {
        make_block<cf64, 4, 128, 2, 4, false>(),          // block: NB 128, R 512, 8 KB runs, cached
        make_set<cf64, 8, 8, 8, false, true>(),           // tiles: NB 64, R 512, cached, x in LDS
        make_block<cf64, 4, 128, 2, 4, true>(),           // block: NB 128, R 512, 8 KB runs
        make_set<cf64, 4, 8, 8, true, false>(),           // tiles: NB 32, R 512
        make_runs<cf64, 4, 16, 8, false, true>(),         // runs: NB 64, R 512, cached, prefetch
        make_strip<cf64, 4, 2, 4, true>(),                // strip: R 512, 8 KB runs, G 4
        make_strip<cf64, 4, 2, 4, false>(),               // strip: R 512, 8 KB runs, G 4, cached
        make_strip<cf64, 8, 1, 4, true>(),                // strip: R 512, 8 KB runs, G 4
        make_strip<cf64, 4, 1, 4, true>(),                // strip: R 256, 4 KB runs, G 4
        make_strip<cf64, 4, 4, 4, false>(),               // strip: R 1024, 16 KB runs, G 4, cached
        make_strip<cf64, 8, 2, 4, true>(),                // strip: R 1024, 16 KB runs, G 4
        make_strip<cf64, 4, 4, 4, true>(),                // strip: R 1024, 16 KB runs, G 4
        make_strip<cf64, 16, 2, 4, true, 1>(),            // strip: R 2048, 32 KB runs, G 4, split by stored rows
        make_strip<cf64, 8, 2, 4, true, 1>(),             // strip: R 1024, 16 KB runs, G 4, split by stored rows
        make_strip<cf64, 16, 1, 8, true, 1>(),            // strip: R 1024, 16 KB runs, G 8, split by stored rows
        make_strip<cf64, 16, 2, 4, true, 2>(),            // strip: R 2048, 32 KB runs, G 4, split by height alone
        make_strip<cf64, 16, 1, 8, true, 2>(),            // strip: R 1024, 16 KB runs, G 8, split by height alone
    };
    return v;
}

template <>
int autotune_for<cf64>(char uplo, int n, int lda, int reps, hipStream_t stream, int* best_idx,
                      float* ms, int max_cfg)
{
    return autotune_impl<cf64>(uplo, n, lda, reps, stream, best_idx, ms, max_cfg);
}

// xGEMV configurations (the built-in choice per transposition and size is
// gemv_defaults below; xgemv_select_config forces one)
template <> const std::vector<GemvKernelSet<cf64>>& gemv_kernel_sets<cf64>()
{
    static const std::vector<GemvKernelSet<cf64>> v = {
        make_gemv<cf64, 16, 1, 8, true>(),                 // R 1024, 16 KB runs, G 8
        make_gemv<cf64, 16, 2, 4, true>(),                 // R 2048, 32 KB runs, G 4
        make_gemv<cf64, 8, 2, 4, true>(),                  // R 1024, 16 KB runs, G 4
    };
    return v;
}

// built-in choice [0 'N', 1 'T' or 'C'][size class]: the fastest (four passes
// of 20 flushed calls, tuned/mi355x_level2.json) at the orders 8192, 16384,
// 23170 on MI355X
template <> GemvDefaults gemv_defaults<cf64>()
{
    return GemvDefaults{{{2, 0, 2}, {2, 0, 2}}};
}

// xSYR2 / xHER2 configurations (the built-in choice per triangle and size is
// syr2_defaults below; xsyr2_select_config forces one)
template <> const std::vector<Syr2KernelSet<cf64>>& syr2_kernel_sets<cf64>()
{
    static const std::vector<Syr2KernelSet<cf64>> v = {
        make_syr2<cf64, 16, 1, 4, true, 1>(),              // R 1024, 16 KB runs, G 4
        make_syr2<cf64, 8, 2, 4, true, 1>(),               // R 1024, 16 KB runs, G 4
        make_syr2<cf64, 4, 2, 4, true, 0>(),               // R 512, 8 KB runs, G 4
    };
    return v;
}

// built-in choice [upper][size class]: the fastest (four passes of 20 flushed
// calls, tuned/mi355x_level2.json) at the orders 8192, 16384 and 23170 on
// MI355X
template <> Syr2Defaults syr2_defaults<cf64>() { return Syr2Defaults{{{0, 0, 1}, {0, 1, 1}}}; }

// xTRMV configurations (xtrmv_select_config forces one; otherwise
// trmv_defaults picks per triangle, transposition and size)
template <> const std::vector<TrmvKernelSet<cf64>>& trmv_kernel_sets<cf64>()
{
    static const std::vector<TrmvKernelSet<cf64>> v = {
        make_trmv<cf64, 16, 1, 4, true, 1>(),              // R 1024, 16 KB runs, G 4, split by stored rows
        make_trmv<cf64, 8, 2, 4, true, 1>(),               // R 1024, 16 KB runs, G 4, split by stored rows
        make_trmv<cf64, 4, 2, 4, true, 0>(),               // R 512, 8 KB runs, G 4
        make_trmv<cf64, 16, 1, 4, true, 0>(),              // R 1024, 16 KB runs, G 4
        make_trmv<cf64, 16, 1, 8, true, 1>(),              // R 1024, 16 KB runs, G 8, split by stored rows
    };
    return v;
}

// built-in choice [upper][0 'N', 1 'T' or 'C'][size class]: the fastest (four
// passes of 20 flushed calls, tuned/mi355x_level2.json; 'T' and 'C' by their
// summed time) at the orders 8192, 16384 and 23170 on MI355X
template <> TrmvDefaults trmv_defaults<cf64>()
{
    return TrmvDefaults{{{{4, 4, 0}, {4, 4, 0}}, {{0, 4, 1}, {1, 3, 1}}}};
}

// One shard's product: the row-strip shape that the built-in rules pick for
// the largest orders (R 2048, G 4, split by stored rows)
template <> const ShardKernelSet<cf64>& shard_kernels<cf64>()
{
    static const ShardKernelSet<cf64> k = make_shard<cf64, 16, 2, 4, true, 1>();
    return k;
}
}  // namespace xsymv

extern "C" int xhemv_z(char uplo, int n, xcomplex128 alpha, const xcomplex128* A, int lda,
                       const xcomplex128* x, int incx, xcomplex128 beta, xcomplex128* y,
                       int incy,
                       void* stream)
{
    using xsymv::cf64;
    return xsymv::symv_impl<cf64>(uplo, n, cf64{alpha.re, alpha.im}, (const cf64*)A, lda,
                                  (const cf64*)x, incx, cf64{beta.re, beta.im}, (cf64*)y, incy,
                                  (hipStream_t)stream);
}

extern "C" int xgemv_z(char trans, int m, int n, xcomplex128 alpha, const xcomplex128* A, int lda,
                       const xcomplex128* x, int incx, xcomplex128 beta, xcomplex128* y, int incy,
                       void* stream)
{
    using xsymv::cf64;
    return xsymv::gemv_run<cf64>(trans, m, n, cf64{alpha.re, alpha.im},
                               reinterpret_cast<const cf64*>(A), lda,
                               reinterpret_cast<const cf64*>(x), incx, cf64{beta.re, beta.im},
                               reinterpret_cast<cf64*>(y), incy, (hipStream_t)stream, -1);
}

extern "C" int xher2_z(char uplo, int n, xcomplex128 alpha, const xcomplex128* x, int incx, const xcomplex128* y,
                       int incy, xcomplex128* A, int lda, void* stream)
{
    using xsymv::cf64;
    return xsymv::syr2_run<cf64>(uplo, n, cf64{alpha.re, alpha.im}, (const cf64*)x, incx,
                               (const cf64*)y, incy, (cf64*)A, lda, (hipStream_t)stream, -1);
}

extern "C" int xtrmv_z(char uplo, char trans, char diag, int n, const xcomplex128* A, int lda,
                       xcomplex128* x, int incx, void* stream)
{
    using xsymv::cf64;
    return xsymv::trmv_run<cf64>(uplo, trans, diag, n, (const cf64*)A, lda, (cf64*)x, incx,
                               (hipStream_t)stream, -1);
}

extern "C" int xhemv_shard_z(char uplo, int n, int panel, int nshards, int shard,
                            const xcomplex128* Aloc, int lda, const xcomplex128* x, int incx, xcomplex128* p,
                            void* stream)
{
    using xsymv::cf64;
    return xsymv::shard_run<cf64>(uplo, n, panel, nshards, shard, (const cf64*)Aloc, lda,
                                    (const cf64*)x, incx, (cf64*)p, (hipStream_t)stream);
}

extern "C" int xhemv_combine_z(int n, int nshards, xcomplex128 alpha, const xcomplex128* P, int ldp,
                              xcomplex128 beta, xcomplex128* y, int incy, void* stream)
{
    using xsymv::cf64;
    return xsymv::combine_run<cf64>(n, nshards, cf64{alpha.re, alpha.im}, (const cf64*)P, ldp,
                                      cf64{beta.re, beta.im}, (cf64*)y, incy, (hipStream_t)stream);
}
