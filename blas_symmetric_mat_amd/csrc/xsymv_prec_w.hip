// WSYMV (double-double) kernels and entry point of libxsymv.
#include "xsymv_host.hpp"

namespace xsymv {
template <> const std::vector<KernelSet<ddreal>>& kernel_sets<ddreal>()
{
    // index 0 is the built-in default (fastest streaming kernel measured on MI355X
    // at the largest benchmark size of this precision)
    static const std::vector<KernelSet<ddreal>> v = {
        make_set<ddreal, 4, 8, 4, true, false>(),         // tiles: NB 32, R 256
        make_runs<ddreal, 4, 16, 8, true, true>(),        // runs: NB 64, R 512, prefetch
        make_block<ddreal, 4, 64, 2, 4, true>(),          // block: NB 64, R 512, 8 KB runs
        make_set<ddreal, 8, 8, 4, true, false>(),         // tiles: NB 64, R 256
        make_block<ddreal, 4, 128, 2, 4, true>(),         // block: NB 128, R 512, 8 KB runs
        make_strip<ddreal, 4, 2, 4, true>(),              // strip: R 512, 8 KB runs, G 4
        make_strip<ddreal, 4, 2, 4, false>(),             // strip: R 512, 8 KB runs, G 4, cached
        make_strip<ddreal, 8, 1, 4, true>(),              // strip: R 512, 8 KB runs, G 4
        make_strip<ddreal, 4, 1, 4, true>(),              // strip: R 256, 4 KB runs, G 4
        make_strip<ddreal, 4, 2, 2, true>(),              // strip: R 512, 8 KB runs, G 2
        make_strip<ddreal, 8, 2, 4, true>(),              // strip: R 1024, 16 KB runs, G 4
        make_strip<ddreal, 4, 4, 4, true>(),              // strip: R 1024, 16 KB runs, G 4
        make_strip<ddreal, 16, 2, 4, true, 1>(),          // strip: R 2048, 32 KB runs, G 4, split by stored rows
        make_strip<ddreal, 4, 4, 4, true, 1>(),           // strip: R 1024, 16 KB runs, G 4, split by stored rows
        make_strip<ddreal, 16, 1, 4, true, 1>(),          // strip: R 1024, 16 KB runs, G 4, split by stored rows
        make_strip<ddreal, 8, 2, 4, true>(),              // strip: R 1024, 16 KB runs, G 4
        make_strip<ddreal, 4, 4, 4, true, 2>(),           // strip: R 1024, 16 KB runs, G 4, split by height alone
        make_strip<ddreal, 4, 2, 4, true, 2>(),           // strip: R 512, 8 KB runs, G 4, split by height alone
        make_strip<ddreal, 16, 1, 4, true, 2>(),          // strip: R 1024, 16 KB runs, G 4, split by height alone
    };
    return v;
}

template <>
int autotune_for<ddreal>(char uplo, int n, int lda, int reps, hipStream_t stream, int* best_idx,
                      float* ms, int max_cfg)
{
    return autotune_impl<ddreal>(uplo, n, lda, reps, stream, best_idx, ms, max_cfg);
}

// xGEMV configurations (the built-in choice per transposition and size is
// gemv_defaults below; xgemv_select_config forces one)
template <> const std::vector<GemvKernelSet<ddreal>>& gemv_kernel_sets<ddreal>()
{
    static const std::vector<GemvKernelSet<ddreal>> v = {
        make_gemv<ddreal, 8, 2, 4, true>(),                // R 1024, 16 KB runs, G 4
        make_gemv<ddreal, 4, 4, 4, true>(),                // R 1024, 16 KB runs, G 4
        make_gemv<ddreal, 16, 1, 4, true>(),               // R 1024, 16 KB runs, G 4
    };
    return v;
}

// built-in choice [0 'N', 1 'T'][size class]: the fastest (four passes of 20
// flushed calls, tuned/mi355x_level2.json) at the orders 8192, 16384, 23170 on
// MI355X
template <> GemvDefaults gemv_defaults<ddreal>()
{
    return GemvDefaults{{{2, 1, 1}, {1, 1, 1}}};
}

// xSYR2 / xHER2 configurations (the built-in choice per triangle and size is
// syr2_defaults below; xsyr2_select_config forces one)
template <> const std::vector<Syr2KernelSet<ddreal>>& syr2_kernel_sets<ddreal>()
{
    static const std::vector<Syr2KernelSet<ddreal>> v = {
        make_syr2<ddreal, 16, 1, 4, true, 1>(),            // R 1024, 16 KB runs, G 4
        make_syr2<ddreal, 8, 2, 4, true, 1>(),             // R 1024, 16 KB runs, G 4
        make_syr2<ddreal, 4, 2, 4, true, 0>(),             // R 512, 8 KB runs, G 4
    };
    return v;
}

// built-in choice [upper][size class]: the fastest (four passes of 20 flushed
// calls, tuned/mi355x_level2.json) at the orders 8192, 16384 and 23170 on
// MI355X
template <> Syr2Defaults syr2_defaults<ddreal>() { return Syr2Defaults{{{0, 2, 1}, {0, 1, 1}}}; }

// xTRMV configurations (xtrmv_select_config forces one; otherwise
// trmv_defaults picks per triangle, transposition and size)
template <> const std::vector<TrmvKernelSet<ddreal>>& trmv_kernel_sets<ddreal>()
{
    static const std::vector<TrmvKernelSet<ddreal>> v = {
        make_trmv<ddreal, 16, 1, 4, true, 1>(),            // R 1024, 16 KB runs, G 4, split by stored rows
        make_trmv<ddreal, 8, 2, 4, true, 1>(),             // R 1024, 16 KB runs, G 4, split by stored rows
        make_trmv<ddreal, 4, 2, 4, true, 0>(),             // R 512, 8 KB runs, G 4
        make_trmv<ddreal, 16, 1, 4, true, 0>(),            // R 1024, 16 KB runs, G 4
        make_trmv<ddreal, 16, 1, 8, true, 1>(),            // R 1024, 16 KB runs, G 8, split by stored rows
    };
    return v;
}

// built-in choice [upper][0 'N', 1 'T'][size class]: the fastest (four passes
// of 20 flushed calls, tuned/mi355x_level2.json; 'T' and 'C' by their summed
// time) at the orders 8192, 16384 and 23170 on MI355X
template <> TrmvDefaults trmv_defaults<ddreal>()
{
    return TrmvDefaults{{{{4, 4, 4}, {2, 2, 4}}, {{4, 4, 4}, {1, 4, 1}}}};
}

// One shard's product: the row-strip shape that the built-in rules pick for
// the largest orders (R 1024, G 4, split by strip height)
template <> const ShardKernelSet<ddreal>& shard_kernels<ddreal>()
{
    static const ShardKernelSet<ddreal> k = make_shard<ddreal, 4, 4, 4, true, 0>();
    return k;
}
}  // namespace xsymv

extern "C" int xsymv_w(char uplo, int n, xdd alpha, const xdd* A, int lda, const xdd* x,
                       int incx, xdd beta, xdd* y, int incy,
                       void* stream)
{
    using xsymv::ddreal;
    return xsymv::symv_impl<ddreal>(uplo, n, ddreal{alpha.hi, alpha.lo}, (const ddreal*)A, lda,
                                    (const ddreal*)x, incx, ddreal{beta.hi, beta.lo},
                                    (ddreal*)y, incy, (hipStream_t)stream);
}

extern "C" int xgemv_w(char trans, int m, int n, xdd alpha, const xdd* A, int lda,
                       const xdd* x, int incx, xdd beta, xdd* y, int incy,
                       void* stream)
{
    using xsymv::ddreal;
    return xsymv::gemv_run<ddreal>(trans, m, n, ddreal{alpha.hi, alpha.lo},
                               reinterpret_cast<const ddreal*>(A), lda,
                               reinterpret_cast<const ddreal*>(x), incx, ddreal{beta.hi, beta.lo},
                               reinterpret_cast<ddreal*>(y), incy, (hipStream_t)stream, -1);
}

extern "C" int xsyr2_w(char uplo, int n, xdd alpha, const xdd* x, int incx, const xdd* y,
                       int incy, xdd* A, int lda, void* stream)
{
    using xsymv::ddreal;
    return xsymv::syr2_run<ddreal>(uplo, n, ddreal{alpha.hi, alpha.lo}, (const ddreal*)x, incx,
                               (const ddreal*)y, incy, (ddreal*)A, lda, (hipStream_t)stream, -1);
}

extern "C" int xtrmv_w(char uplo, char trans, char diag, int n, const xdd* A, int lda, xdd* x,
                       int incx, void* stream)
{
    using xsymv::ddreal;
    return xsymv::trmv_run<ddreal>(uplo, trans, diag, n, (const ddreal*)A, lda, (ddreal*)x, incx,
                                   (hipStream_t)stream, -1);
}

extern "C" int xsymv_shard_w(char uplo, int n, int panel, int nshards, int shard,
                            const xdd* Aloc, int lda, const xdd* x, int incx, xdd* p,
                            void* stream)
{
    using xsymv::ddreal;
    return xsymv::shard_run<ddreal>(uplo, n, panel, nshards, shard, (const ddreal*)Aloc, lda,
                                    (const ddreal*)x, incx, (ddreal*)p, (hipStream_t)stream);
}

extern "C" int xsymv_combine_w(int n, int nshards, xdd alpha, const xdd* P, int ldp,
                              xdd beta, xdd* y, int incy, void* stream)
{
    using xsymv::ddreal;
    return xsymv::combine_run<ddreal>(n, nshards, ddreal{alpha.hi, alpha.lo}, (const ddreal*)P, ldp,
                                      ddreal{beta.hi, beta.lo}, (ddreal*)y, incy, (hipStream_t)stream);
}
