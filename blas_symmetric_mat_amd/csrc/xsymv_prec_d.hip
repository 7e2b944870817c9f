// DSYMV (double) kernels and entry point of libxsymv.
#include "xsymv_host.hpp"

namespace xsymv {
template <> const std::vector<KernelSet<double>>& kernel_sets<double>()
{
    // index 0 is the built-in default (fastest streaming kernel measured on MI355X
    // at the largest benchmark size of this precision)
    static const std::vector<KernelSet<double>> v = {
        make_block<double, 4, 128, 2, 4, false>(),        // block: NB 128, R 1024, 8 KB runs, cached
        make_block<double, 4, 256, 2, 4, true>(),         // block: NB 256, R 1024, 8 KB runs
        make_set<double, 4, 16, 4, false, false>(),       // tiles: NB 64, R 512, cached
        make_runs<double, 4, 16, 8, true, true>(),        // runs: NB 64, R 1024, prefetch
        make_block<double, 4, 128, 2, 4, true>(),         // block: NB 128, R 1024, 8 KB runs
        make_set<double, 8, 16, 2, false, false>(),       // tiles: NB 128, R 256, cached
        make_strip<double, 4, 2, 4, true>(),              // strip: R 1024, 8 KB runs, G 4
        make_strip<double, 4, 2, 4, false>(),             // strip: R 1024, 8 KB runs, G 4, cached
        make_strip<double, 4, 2, 8, true>(),              // strip: R 1024, 8 KB runs, G 8
        make_strip<double, 8, 1, 4, true>(),              // strip: R 1024, 8 KB runs, G 4
        make_strip<double, 4, 1, 4, true>(),              // strip: R 512, 4 KB runs, G 4
        make_strip<double, 4, 4, 4, false>(),             // strip: R 2048, 16 KB runs, G 4, cached
        make_strip<double, 4, 2, 8, false>(),             // strip: R 1024, 8 KB runs, G 8, cached
        make_strip<double, 8, 2, 4, true>(),              // strip: R 2048, 16 KB runs, G 4
        make_strip<double, 8, 1, 8, true>(),              // strip: R 1024, 8 KB runs, G 8
        make_strip<double, 16, 2, 4, true, 1>(),          // strip: R 4096, 32 KB runs, G 4, split by stored rows
        make_strip<double, 16, 1, 4, true, 1>(),          // strip: R 2048, 16 KB runs, G 4, split by stored rows
        make_strip<double, 8, 2, 4, true, 1>(),           // strip: R 2048, 16 KB runs, G 4, split by stored rows
        make_strip<double, 8, 1, 8, true, 1>(),           // strip: R 1024, 8 KB runs, G 8, split by stored rows
        make_strip<double, 16, 2, 8, true, 1>(),          // strip: R 4096, 32 KB runs, G 8, split by stored rows
        make_strip<double, 16, 1, 16, true, 1>(),         // strip: R 2048, 16 KB runs, G 16, split by stored rows
        make_strip<double, 16, 1, 8, true, 1>(),          // strip: R 2048, 16 KB runs, G 8, split by stored rows
        make_strip<double, 8, 1, 8, true, 2>(),           // strip: R 1024, 8 KB runs, G 8, split by height alone
        make_strip<double, 16, 1, 8, true, 2>(),          // strip: R 2048, 16 KB runs, G 8, split by height alone
    };
    return v;
}

template <>
int autotune_for<double>(char uplo, int n, int lda, int reps, hipStream_t stream, int* best_idx,
                      float* ms, int max_cfg)
{
    return autotune_impl<double>(uplo, n, lda, reps, stream, best_idx, ms, max_cfg);
}

// xGEMV configurations (the built-in choice per transposition and size is
// gemv_defaults below; xgemv_select_config forces one)
template <> const std::vector<GemvKernelSet<double>>& gemv_kernel_sets<double>()
{
    static const std::vector<GemvKernelSet<double>> v = {
        make_gemv<double, 16, 1, 8, true>(),               // R 2048, 16 KB runs, G 8
        make_gemv<double, 16, 2, 4, true>(),               // R 4096, 32 KB runs, G 4
        make_gemv<double, 16, 1, 16, true>(),              // R 2048, 16 KB runs, G 16
        make_gemv<double, 8, 2, 8, true>(),                // R 2048, 16 KB runs, G 8
    };
    return v;
}

// built-in choice [0 'N', 1 'T'][size class]: the fastest (four passes of 20
// flushed calls, tuned/mi355x_level2.json) at the orders 8192, 16384, 32768 on
// MI355X
template <> GemvDefaults gemv_defaults<double>()
{
    return GemvDefaults{{{2, 3, 2}, {0, 3, 2}}};
}

// xSYR2 / xHER2 configurations (the built-in choice per triangle and size is
// syr2_defaults below; xsyr2_select_config forces one)
template <> const std::vector<Syr2KernelSet<double>>& syr2_kernel_sets<double>()
{
    static const std::vector<Syr2KernelSet<double>> v = {
        make_syr2<double, 16, 1, 4, true, 1>(),            // R 2048, 16 KB runs, G 4
        make_syr2<double, 16, 2, 4, true, 1>(),            // R 4096, 32 KB runs, G 4
        make_syr2<double, 8, 2, 4, true, 1>(),             // R 2048, 16 KB runs, G 4
        make_syr2<double, 4, 2, 4, true, 0>(),             // R 1024, 8 KB runs, G 4
    };
    return v;
}

// built-in choice [upper][size class]: the fastest (four passes of 20 flushed
// calls, tuned/mi355x_level2.json) at the orders 8192, 16384 and 32768 on
// MI355X
template <> Syr2Defaults syr2_defaults<double>() { return Syr2Defaults{{{0, 0, 0}, {0, 1, 2}}}; }

// xTRMV configurations (xtrmv_select_config forces one; otherwise
// trmv_defaults picks per triangle, transposition and size)
template <> const std::vector<TrmvKernelSet<double>>& trmv_kernel_sets<double>()
{
    static const std::vector<TrmvKernelSet<double>> v = {
        make_trmv<double, 16, 1, 8, true, 1>(),            // R 2048, 16 KB runs, G 8, split by stored rows
        make_trmv<double, 16, 1, 4, true, 1>(),            // R 2048, 16 KB runs, G 4, split by stored rows
        make_trmv<double, 8, 2, 4, true, 0>(),             // R 2048, 16 KB runs, G 4
        make_trmv<double, 16, 1, 4, true, 0>(),            // R 2048, 16 KB runs, G 4
        make_trmv<double, 16, 2, 4, true, 1>(),            // R 4096, 32 KB runs, G 4, split by stored rows
        make_trmv<double, 8, 2, 8, true, 1>(),             // R 2048, 16 KB runs, G 8, split by stored rows
    };
    return v;
}

// built-in choice [upper][0 'N', 1 'T'][size class]: the fastest (four passes
// of 20 flushed calls, tuned/mi355x_level2.json; 'T' and 'C' by their summed
// time) at the orders 8192, 16384 and 32768 on MI355X
template <> TrmvDefaults trmv_defaults<double>()
{
    return TrmvDefaults{{{{0, 1, 0}, {1, 1, 3}}, {{0, 1, 0}, {5, 3, 3}}}};
}

// One shard's product (537 MB at n = 32768 with 8 shards): R 2048, G 8,
// split by strip height alone -- the fastest of five shapes measured on the
// per-GPU share at that order
template <> const ShardKernelSet<double>& shard_kernels<double>()
{
    static const ShardKernelSet<double> k = make_shard<double, 16, 1, 8, true, 2>();
    return k;
}
}  // namespace xsymv

extern "C" int xsymv_d(char uplo, int n, double alpha, const double* A, int lda,
                       const double* x, int incx, double beta, double* y, int incy,
                       void* stream)
{
    return xsymv::symv_impl<double>(uplo, n, alpha, A, lda, x, incx, beta, y, incy,
                                    (hipStream_t)stream);
}

extern "C" int xgemv_d(char trans, int m, int n, double alpha, const double* A, int lda,
                       const double* x, int incx, double beta, double* y, int incy, void* stream)
{
    return xsymv::gemv_run<double>(trans, m, n, alpha, A, lda, x, incx, beta, y, incy,
                               (hipStream_t)stream, -1);
}

extern "C" int xsyr2_d(char uplo, int n, double alpha, const double* x, int incx, const double* y,
                       int incy, double* A, int lda, void* stream)
{
    return xsymv::syr2_run<double>(uplo, n, alpha, x, incx, y, incy, A, lda, (hipStream_t)stream,
                               -1);
}

extern "C" int xtrmv_d(char uplo, char trans, char diag, int n, const double* A, int lda, double* x,
                       int incx, void* stream)
{
    return xsymv::trmv_run<double>(uplo, trans, diag, n, A, lda, x, incx, (hipStream_t)stream, -1);
}

extern "C" int xsymv_shard_d(char uplo, int n, int panel, int nshards, int shard,
                            const double* Aloc, int lda, const double* x, int incx, double* p,
                            void* stream)
{
    return xsymv::shard_run<double>(uplo, n, panel, nshards, shard, Aloc, lda, x, incx, p,
                                    (hipStream_t)stream);
}

extern "C" int xsymv_combine_d(int n, int nshards, double alpha, const double* P, int ldp,
                              double beta, double* y, int incy, void* stream)
{
    return xsymv::combine_run<double>(n, nshards, alpha, P, ldp, beta, y, incy, (hipStream_t)stream);
}
