// SSYMV (float) kernels and entry point of libxsymv.
#include "xsymv_host.hpp"

namespace xsymv {
template <> const std::vector<KernelSet<float>>& kernel_sets<float>()
{
    // index 0 is the built-in default (fastest streaming kernel measured on MI355X
    // at the largest benchmark size of this precision)
    static const std::vector<KernelSet<float>> v = {
        make_set<float, 8, 16, 2, true, false>(),         // tiles: NB 128, R 512
        make_block<float, 4, 128, 2, 4, true>(),          // block: NB 128, R 2048, 8 KB runs
        make_set<float, 4, 16, 4, true, false>(),         // tiles: NB 64, R 1024
        make_block<float, 4, 64, 2, 4, true>(),           // block: NB 64, R 2048, 8 KB runs
        make_block<float, 8, 128, 1, 4, true>(),          // block: NB 128, R 2048, 8 KB runs
        make_runs<float, 4, 16, 8, true, true>(),         // runs: NB 64, R 2048, prefetch
        make_strip<float, 4, 2, 4, true>(),               // strip: R 2048, 8 KB runs, G 4
        make_strip<float, 4, 2, 4, false>(),              // strip: R 2048, 8 KB runs, G 4, cached
        make_strip<float, 4, 2, 8, true>(),               // strip: R 2048, 8 KB runs, G 8
        make_strip<float, 8, 1, 4, true>(),               // strip: R 2048, 8 KB runs, G 4
        make_strip<float, 4, 1, 4, true>(),               // strip: R 1024, 4 KB runs, G 4
        make_strip<float, 4, 4, 4, true>(),               // strip: R 4096, 16 KB runs, G 4
        make_strip<float, 8, 2, 4, true>(),               // strip: R 4096, 16 KB runs, G 4
        make_strip<float, 16, 1, 4, true>(),              // strip: R 4096, 16 KB runs, G 4
        make_strip<float, 16, 1, 4, true, 1>(),           // strip: R 4096, 16 KB runs, G 4, split by stored rows
        make_strip<float, 8, 1, 4, true, 1>(),            // strip: R 2048, 8 KB runs, G 4, split by stored rows
        make_strip<float, 4, 2, 8, true, 1>(),            // strip: R 2048, 8 KB runs, G 8, split by stored rows
        make_strip<float, 16, 1, 16, true>(),             // strip: R 4096, 16 KB runs, G 16
        make_strip<float, 16, 1, 16, true, 1>(),          // strip: R 4096, 16 KB runs, G 16, split by stored rows
        make_strip<float, 16, 1, 8, true>(),              // strip: R 4096, 16 KB runs, G 8
        make_strip<float, 16, 2, 8, true, 1>(),           // strip: R 8192, 32 KB runs, G 8, split by stored rows
        make_strip<float, 8, 4, 4, true, 1>(),            // strip: R 8192, 32 KB runs, G 4, split by stored rows
        make_strip<float, 16, 1, 16, true, 2>(),          // strip: R 4096, 16 KB runs, G 16, split by height alone
    };
    return v;
}

template <>
int autotune_for<float>(char uplo, int n, int lda, int reps, hipStream_t stream, int* best_idx,
                      float* ms, int max_cfg)
{
    return autotune_impl<float>(uplo, n, lda, reps, stream, best_idx, ms, max_cfg);
}

// xGEMV configurations (the built-in choice per transposition and size is
// gemv_defaults below; xgemv_select_config forces one)
template <> const std::vector<GemvKernelSet<float>>& gemv_kernel_sets<float>()
{
    static const std::vector<GemvKernelSet<float>> v = {
        make_gemv<float, 16, 2, 4, true>(),                // R 8192, 32 KB runs, G 4
        make_gemv<float, 16, 1, 8, true>(),                // R 4096, 16 KB runs, G 8
        make_gemv<float, 16, 1, 16, true>(),               // R 4096, 16 KB runs, G 16
        make_gemv<float, 8, 2, 8, true>(),                 // R 4096, 16 KB runs, G 8
    };
    return v;
}

// built-in choice [0 'N', 1 'T'][size class]: the fastest (four passes of 20
// flushed calls, tuned/mi355x_level2.json) at the orders 8192, 16384, 32768 on
// MI355X
template <> GemvDefaults gemv_defaults<float>()
{
    return GemvDefaults{{{1, 1, 2}, {1, 1, 0}}};
}

// xSYR2 / xHER2 configurations (the built-in choice per triangle and size is
// syr2_defaults below; xsyr2_select_config forces one)
template <> const std::vector<Syr2KernelSet<float>>& syr2_kernel_sets<float>()
{
    static const std::vector<Syr2KernelSet<float>> v = {
        make_syr2<float, 16, 1, 16, true, 1>(),            // R 4096, 16 KB runs, G 16
        make_syr2<float, 16, 1, 8, true, 1>(),             // R 4096, 16 KB runs, G 8
        make_syr2<float, 16, 1, 4, true, 1>(),             // R 4096, 16 KB runs, G 4
        make_syr2<float, 8, 2, 4, true, 1>(),              // R 4096, 16 KB runs, G 4
        make_syr2<float, 4, 2, 4, true, 0>(),              // R 2048, 8 KB runs, G 4
        make_syr2<float, 16, 1, 8, true, 2>(),             // R 4096, 16 KB runs, G 8, split by height alone
    };
    return v;
}

// built-in choice [upper][size class]: the fastest (four passes of 20 flushed
// calls, tuned/mi355x_level2.json) at the orders 8192, 16384 and 32768 on
// MI355X
template <> Syr2Defaults syr2_defaults<float>() { return Syr2Defaults{{{5, 5, 5}, {0, 0, 0}}}; }

// xTRMV configurations (xtrmv_select_config forces one; otherwise
// trmv_defaults picks per triangle, transposition and size)
template <> const std::vector<TrmvKernelSet<float>>& trmv_kernel_sets<float>()
{
    static const std::vector<TrmvKernelSet<float>> v = {
        make_trmv<float, 16, 1, 16, true, 1>(),            // R 4096, 16 KB runs, G 16, split by stored rows
        make_trmv<float, 16, 1, 8, true, 1>(),             // R 4096, 16 KB runs, G 8, split by stored rows
        make_trmv<float, 16, 1, 4, true, 0>(),             // R 4096, 16 KB runs, G 4
        make_trmv<float, 16, 1, 4, true, 1>(),             // R 4096, 16 KB runs, G 4, split by stored rows
        make_trmv<float, 8, 2, 4, true, 1>(),              // R 4096, 16 KB runs, G 4, split by stored rows
        make_trmv<float, 16, 2, 4, true, 1>(),             // R 8192, 32 KB runs, G 4, split by stored rows
    };
    return v;
}

// built-in choice [upper][0 'N', 1 'T'][size class]: the fastest (four passes
// of 20 flushed calls, tuned/mi355x_level2.json; 'T' and 'C' by their summed
// time) at the orders 8192, 16384 and 32768 on MI355X
template <> TrmvDefaults trmv_defaults<float>()
{
    return TrmvDefaults{{{{0, 0, 0}, {2, 3, 3}}, {{0, 0, 0}, {4, 4, 5}}}};
}

// One shard's product (268 MB at n = 32768 with 8 shards): R 4096, G 16,
// split by strip height alone -- the fastest of five shapes measured on the
// per-GPU share at that order
template <> const ShardKernelSet<float>& shard_kernels<float>()
{
    static const ShardKernelSet<float> k = make_shard<float, 16, 1, 16, true, 2>();
    return k;
}
}  // namespace xsymv

extern "C" int xsymv_s(char uplo, int n, float alpha, const float* A, int lda, const float* x,
                       int incx, float beta, float* y, int incy, void* stream)
{
    return xsymv::symv_impl<float>(uplo, n, alpha, A, lda, x, incx, beta, y, incy,
                                   (hipStream_t)stream);
}

extern "C" int xgemv_s(char trans, int m, int n, float alpha, const float* A, int lda,
                       const float* x, int incx, float beta, float* y, int incy, void* stream)
{
    return xsymv::gemv_run<float>(trans, m, n, alpha, A, lda, x, incx, beta, y, incy,
                               (hipStream_t)stream, -1);
}

extern "C" int xsyr2_s(char uplo, int n, float alpha, const float* x, int incx, const float* y,
                       int incy, float* A, int lda, void* stream)
{
    return xsymv::syr2_run<float>(uplo, n, alpha, x, incx, y, incy, A, lda, (hipStream_t)stream,
                               -1);
}

extern "C" int xtrmv_s(char uplo, char trans, char diag, int n, const float* A, int lda, float* x,
                       int incx, void* stream)
{
    return xsymv::trmv_run<float>(uplo, trans, diag, n, A, lda, x, incx, (hipStream_t)stream, -1);
}

extern "C" int xsymv_shard_s(char uplo, int n, int panel, int nshards, int shard,
                            const float* Aloc, int lda, const float* x, int incx, float* p,
                            void* stream)
{
    return xsymv::shard_run<float>(uplo, n, panel, nshards, shard, Aloc, lda, x, incx, p,
                                    (hipStream_t)stream);
}

extern "C" int xsymv_combine_s(int n, int nshards, float alpha, const float* P, int ldp,
                              float beta, float* y, int incy, void* stream)
{
    return xsymv::combine_run<float>(n, nshards, alpha, P, ldp, beta, y, incy, (hipStream_t)stream);
}
