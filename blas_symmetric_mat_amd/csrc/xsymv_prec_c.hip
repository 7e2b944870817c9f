// CHEMV (complex float, Hermitian) kernels and entry point of libxsymv.
#include "xsymv_host.hpp"

namespace xsymv {
template <> const std::vector<KernelSet<cf32>>& kernel_sets<cf32>()
{
    // index 0 is the built-in default (fastest streaming kernel measured on MI355X
    // at the largest benchmark size of this precision)
    static const std::vector<KernelSet<cf32>> v = {
        make_set<cf32, 8, 16, 4, true, false>(),          // tiles: NB 128, R 512
        make_block<cf32, 8, 128, 1, 4, true>(),           // block: NB 128, R 1024, 8 KB runs
        make_block<cf32, 4, 128, 2, 4, true>(),           // block: NB 128, R 1024, 8 KB runs
        make_set<cf32, 4, 16, 4, true, false>(),          // tiles: NB 64, R 512
        make_runs<cf32, 4, 16, 8, true, true>(),          // runs: NB 64, R 1024, prefetch
        make_strip<cf32, 4, 2, 4, true>(),                // strip: R 1024, 8 KB runs, G 4
        make_strip<cf32, 4, 2, 4, false>(),               // strip: R 1024, 8 KB runs, G 4, cached
        make_strip<cf32, 8, 1, 4, true>(),                // strip: R 1024, 8 KB runs, G 4
        make_strip<cf32, 4, 1, 4, true>(),                // strip: R 512, 4 KB runs, G 4
        make_strip<cf32, 8, 2, 4, true>(),                // strip: R 2048, 16 KB runs, G 4
        make_strip<cf32, 4, 2, 8, true>(),                // strip: R 1024, 8 KB runs, G 8
        make_strip<cf32, 16, 2, 4, true, 1>(),            // strip: R 4096, 32 KB runs, G 4, split by stored rows
        make_strip<cf32, 8, 2, 4, true, 1>(),             // strip: R 2048, 16 KB runs, G 4, split by stored rows
        make_strip<cf32, 16, 2, 8, true, 1>(),            // strip: R 4096, 32 KB runs, G 8, split by stored rows
        make_strip<cf32, 16, 1, 8, true, 1>(),            // strip: R 2048, 16 KB runs, G 8, split by stored rows
        make_strip<cf32, 16, 1, 8, true, 2>(),            // strip: R 2048, 16 KB runs, G 8, split by height alone
    };
    return v;
}

template <>
int autotune_for<cf32>(char uplo, int n, int lda, int reps, hipStream_t stream, int* best_idx,
                      float* ms, int max_cfg)
{
    return autotune_impl<cf32>(uplo, n, lda, reps, stream, best_idx, ms, max_cfg);
}

// xGEMV configurations (the built-in choice per transposition and size is
// gemv_defaults below; xgemv_select_config forces one)
template <> const std::vector<GemvKernelSet<cf32>>& gemv_kernel_sets<cf32>()
{
    static const std::vector<GemvKernelSet<cf32>> v = {
        make_gemv<cf32, 8, 2, 8, true>(),                  // R 2048, 16 KB runs, G 8
        make_gemv<cf32, 16, 1, 8, true>(),                 // R 2048, 16 KB runs, G 8
        make_gemv<cf32, 16, 2, 4, true>(),                 // R 4096, 32 KB runs, G 4
    };
    return v;
}

// built-in choice [0 'N', 1 'T' or 'C'][size class]: the fastest (four passes
// of 20 flushed calls, tuned/mi355x_level2.json) at the orders 8192, 16384,
// 32768 on MI355X
template <> GemvDefaults gemv_defaults<cf32>()
{
    return GemvDefaults{{{1, 0, 1}, {1, 0, 1}}};
}

// xSYR2 / xHER2 configurations (the built-in choice per triangle and size is
// syr2_defaults below; xsyr2_select_config forces one)
template <> const std::vector<Syr2KernelSet<cf32>>& syr2_kernel_sets<cf32>()
{
    static const std::vector<Syr2KernelSet<cf32>> v = {
        make_syr2<cf32, 16, 1, 4, true, 1>(),              // R 2048, 16 KB runs, G 4
        make_syr2<cf32, 8, 2, 4, true, 1>(),               // R 2048, 16 KB runs, G 4
        make_syr2<cf32, 4, 2, 4, true, 0>(),               // R 1024, 8 KB runs, G 4
    };
    return v;
}

// built-in choice [upper][size class]: the fastest (four passes of 20 flushed
// calls, tuned/mi355x_level2.json) at the orders 8192, 16384 and 32768 on
// MI355X
template <> Syr2Defaults syr2_defaults<cf32>() { return Syr2Defaults{{{2, 0, 0}, {0, 0, 1}}}; }

// xTRMV configurations (xtrmv_select_config forces one; otherwise
// trmv_defaults picks per triangle, transposition and size)
template <> const std::vector<TrmvKernelSet<cf32>>& trmv_kernel_sets<cf32>()
{
    static const std::vector<TrmvKernelSet<cf32>> v = {
        make_trmv<cf32, 16, 1, 8, true, 1>(),              // R 2048, 16 KB runs, G 8, split by stored rows
        make_trmv<cf32, 16, 1, 4, true, 1>(),              // R 2048, 16 KB runs, G 4, split by stored rows
        make_trmv<cf32, 8, 2, 4, true, 0>(),               // R 2048, 16 KB runs, G 4
        make_trmv<cf32, 16, 1, 16, true, 1>(),             // R 2048, 16 KB runs, G 16, split by stored rows
        make_trmv<cf32, 16, 1, 8, true, 0>(),              // R 2048, 16 KB runs, G 8
    };
    return v;
}

// built-in choice [upper][0 'N', 1 'T' or 'C'][size class]: the fastest (four
// passes of 20 flushed calls, tuned/mi355x_level2.json; 'T' and 'C' by their
// summed time) at the orders 8192, 16384 and 32768 on MI355X
template <> TrmvDefaults trmv_defaults<cf32>()
{
    return TrmvDefaults{{{{1, 1, 1}, {1, 0, 3}}, {{3, 3, 3}, {1, 3, 3}}}};
}

// One shard's product: the row-strip shape that the built-in rules pick for
// the largest orders (R 2048, G 8, split by stored rows)
template <> const ShardKernelSet<cf32>& shard_kernels<cf32>()
{
    static const ShardKernelSet<cf32> k = make_shard<cf32, 16, 1, 8, true, 1>();
    return k;
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

extern "C" int xgemv_c(char trans, int m, int n, xcomplex64 alpha, const xcomplex64* A, int lda,
                       const xcomplex64* x, int incx, xcomplex64 beta, xcomplex64* y, int incy,
                       void* stream)
{
    using xsymv::cf32;
    return xsymv::gemv_run<cf32>(trans, m, n, cf32{alpha.re, alpha.im},
                               reinterpret_cast<const cf32*>(A), lda,
                               reinterpret_cast<const cf32*>(x), incx, cf32{beta.re, beta.im},
                               reinterpret_cast<cf32*>(y), incy, (hipStream_t)stream, -1);
}

extern "C" int xher2_c(char uplo, int n, xcomplex64 alpha, const xcomplex64* x, int incx, const xcomplex64* y,
                       int incy, xcomplex64* A, int lda, void* stream)
{
    using xsymv::cf32;
    return xsymv::syr2_run<cf32>(uplo, n, cf32{alpha.re, alpha.im}, (const cf32*)x, incx,
                               (const cf32*)y, incy, (cf32*)A, lda, (hipStream_t)stream, -1);
}

extern "C" int xtrmv_c(char uplo, char trans, char diag, int n, const xcomplex64* A, int lda,
                       xcomplex64* x, int incx, void* stream)
{
    using xsymv::cf32;
    return xsymv::trmv_run<cf32>(uplo, trans, diag, n, (const cf32*)A, lda, (cf32*)x, incx,
                               (hipStream_t)stream, -1);
}

extern "C" int xhemv_shard_c(char uplo, int n, int panel, int nshards, int shard,
                            const xcomplex64* Aloc, int lda, const xcomplex64* x, int incx, xcomplex64* p,
                            void* stream)
{
    using xsymv::cf32;
    return xsymv::shard_run<cf32>(uplo, n, panel, nshards, shard, (const cf32*)Aloc, lda,
                                    (const cf32*)x, incx, (cf32*)p, (hipStream_t)stream);
}

extern "C" int xhemv_combine_c(int n, int nshards, xcomplex64 alpha, const xcomplex64* P, int ldp,
                              xcomplex64 beta, xcomplex64* y, int incy, void* stream)
{
    using xsymv::cf32;
    return xsymv::combine_run<cf32>(n, nshards, cf32{alpha.re, alpha.im}, (const cf32*)P, ldp,
                                      cf32{beta.re, beta.im}, (cf32*)y, incy, (hipStream_t)stream);
}
