// xgemv_strip.hpp -- general matrix-vector product y := alpha*op(A)*x + beta*y
// (op = A, A^T or A^H; A m x n, column-major) on gfx950, on the same
// row-strip harness as the symmetric kernels.
//
// This is the CUDA-xSYMV report's point of comparison: a general product
// reads every element of A once and uses it once, where the symmetric one
// reads one triangle and uses each element twice (report §1, §2.1), so on
// the same streaming machinery GEMV moves twice the bytes of SYMV.
//
//  * Rows are cut into strips of R = W*SW*64*VEC rows; every strip holds all
//    n columns.  The (strip, column) pairs, strip by strip, form one
//    sequence, cut into G equal pieces (G = workgroups the device holds).
//  * Per column, the W waves of a workgroup read one contiguous run of R rows
//    with raw-buffer loads whose byte count ends at row m, so the ragged last
//    strip needs no masks.
//  * 'N': y_i needs the row role only -- each lane keeps SW*VEC row partials
//    in registers for its whole segment and writes them once (no lane
//    exchanges, no LDS, no barriers).
//  * 'T'/'C': y_j needs the column role only -- per group of G columns a
//    halving lane exchange, then the waves are added in wave order through
//    LDS and written to colpart[strip][column].
//  * gemv_merge: y = beta*y + alpha*(partials in a fixed order), no atomics.
#pragma once

#include "xsymv_strip.hpp"

namespace xsymv {

template <class T>
struct GemvArgs {
    const T* A;
    const T* x;           // contiguous: n elements ('N') or m ('T', 'C')
    T* rowpart;           // 'N': [nseg][R]
    T* colpart;           // 'T', 'C': [NS][n]
    const StripBlock* blocks;
    long long lda;
    int m;
    int n;
};

// TR: 0 'N', 1 'T', 2 'C'
template <class T, int TR, int W, int SW, int G, bool NT, int CBUF>
__global__ __launch_bounds__(64 * W) void gemv_strip(GemvArgs<T> a)
{
    using E = Elem<T>;
    constexpr int V = E::VEC;
    constexpr int H = 64 * V;
    constexpr int RW = SW * H;  // rows per wave
    constexpr int R = W * RW;
    constexpr int GROUP = 64 / G;
    static_assert(CBUF % G == 0, "column buffer holds whole groups");

    __shared__ T colred[TR == 0 ? 1 : W][TR == 0 ? 1 : CBUF];

    const StripBlock bd = a.blocks[blockIdx.x];
    const int m = a.m, n = a.n;
    const long long lda = a.lda;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const T* __restrict__ A = a.A;
    const T* __restrict__ x = a.x;
    // 'N': x at a column's index is wave-uniform; for the fp32 types it is
    // read by scalar loads, off the in-order vector-memory counter (as in the
    // symmetric kernels' lower triangle)
    constexpr bool XS = E::SCALAR_X && TR == 0;
    using cword = const __attribute__((address_space(4))) unsigned*;
    const cword xw = (cword)a.x;

    int u = bd.u0;
    int slot = bd.slot0;
    int strip = bd.strip0;
    while (u < bd.u1) {  // workgroup-uniform: one segment per iteration
        const int useg = min(bd.u1, (strip + 1) * n);
        const int rs0 = strip * R;
        const int rs1 = min(m, rs0 + R);
        const int rw = rs0 + wave * RW;  // this wave's first row
        const bool wave_empty = rw >= rs1;
        // this wave's rows of a column: [rw, rw + rows)
        const int rows = min(RW, max(0, m - rw));
        const int coff = -strip * n;  // column = sequence position + coff

        T racc[SW][V];
        T xr[SW][V];
#pragma unroll
        for (int s = 0; s < SW; ++s)
#pragma unroll
            for (int k = 0; k < V; ++k) {
                racc[s][k] = E::zero();
                if (TR != 0) {
                    const int r = rw + s * H + lane * V + k;
                    const T v = x[r < rs1 ? r : rs1 - 1];
                    xr[s][k] = E::sel(r < rs1, v, E::zero());
                }
            }

        int jbuf = u + coff;  // first column held in colred
        int nbuf = 0;         // columns held in colred
#pragma unroll 1
        for (int g0 = u; g0 < useg; g0 += G) {
            const int jg = g0 + coff;          // first column of the group
            const int ng = min(G, useg - g0);  // real columns in the group
            T cacc[G];
#pragma unroll
            for (int g = 0; g < G; ++g) cacc[g] = E::zero();
            // FULL ('N'): every column of the group is real (all groups but a
            // segment's last), so x needs no select and is used by the
            // multiply-adds only; compiled twice where a lane's vector holds
            // several elements
            auto stream_group = [&](auto full) {
                constexpr bool FULL = decltype(full)::value;
                T av[G][SW][V];
                T xcol[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const bool real = FULL || g < ng;
                    const int cc = real ? jg + g : jg;
                    const auto rs = make_rsrc(A + (long long)cc * lda + rw,
                                              (real ? rows : 0) * (int)sizeof(T));
#pragma unroll
                    for (int s = 0; s < SW; ++s)
                        E::template bload16<NT>(rs, (s * H + lane * V) * (int)sizeof(T), av[g][s]);
                    if (TR == 0) {
                        const T xv = XS ? uniform_load<T>(xw, cc) : x[cc];
                        xcol[g] = FULL ? xv : E::sel(real, xv, E::zero());
                    }
                }
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int s = 0; s < SW; ++s)
#pragma unroll
                        for (int k = 0; k < V; ++k) {
                            if (TR == 0)
                                racc[s][k] = E::mac(racc[s][k], av[g][s][k], xcol[g]);
                            else if (TR == 1)
                                cacc[g] = E::mac(cacc[g], av[g][s][k], xr[s][k]);
                            else
                                cacc[g] = E::macc(cacc[g], av[g][s][k], xr[s][k]);
                        }
            };
            if (!wave_empty) {
                if (TR == 0 && V > 1 && ng == G)
                    stream_group(std::integral_constant<bool, (TR == 0 && V > 1)>{});
                else
                    stream_group(std::false_type{});
            }
            if (TR != 0) {
                wave_transpose_reduce<T, G>(cacc, lane);
                if ((lane & (GROUP - 1)) == 0)
                    colred[wave][nbuf + wave_transpose_index<G>(lane)] = cacc[0];
                nbuf += G;
                const bool last = g0 + G >= useg;
                if (nbuf == CBUF || last) {  // workgroup-uniform
                    __syncthreads();
                    const int nreal = last ? (useg - g0) + nbuf - G : nbuf;
                    for (int c = threadIdx.x; c < nreal; c += 64 * W) {
                        T sum = colred[0][c];
#pragma unroll
                        for (int w = 1; w < W; ++w) sum = E::add(sum, colred[w][c]);
                        a.colpart[(long long)strip * n + jbuf + c] = sum;
                    }
                    __syncthreads();
                    jbuf += nreal;
                    nbuf = 0;
                }
            }
        }
        if (TR == 0) {
            T* __restrict__ rp = a.rowpart + (long long)slot * R;
#pragma unroll
            for (int s = 0; s < SW; ++s)
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const int r = rw + s * H + lane * V + k;
                    if (r < rs1) rp[r - rs0] = racc[s][k];
                }
        }
        u = useg;
        ++slot;
        ++strip;
    }
}

// Ordered merge: output o adds its terms k = 0..K-1 (at P[base + k*stride])
// -- 'N': the row partials of o's strip, segment by segment; 'T'/'C': the
// column partials of o over the strips in ascending order.  SPLIT waves
// share 64 outputs; wave g takes the terms k with k % SPLIT == g; the
// subtotals meet in a fixed pairwise tree (the order of symv_strip_merge).
template <class T>
struct GemvMergeArgs {
    const T* part;
    const int* seg_base;  // 'N': segments of strip i are [seg_base[i], seg_base[i+1])
    T* y;
    long long incy;
    long long ky;
    T alpha;
    T beta;
    int leny;
    int NS;
    int R;
    int n;
    int trans;  // 0 'N', else 'T'/'C'
    int beta_zero;
};

template <class T, int SPLIT>
__global__ __launch_bounds__(64 * SPLIT) void gemv_merge(GemvMergeArgs<T> a)
{
    using E = Elem<T>;
    __shared__ T part[SPLIT][64];
    const int lane = threadIdx.x & 63;
    const int g = threadIdx.x >> 6;
    const int o = blockIdx.x * 64 + lane;
    T acc = E::zero();
    if (o < a.leny) {
        long long base, stride;
        int K;
        if (a.trans == 0) {
            const int I = o / a.R;
            K = a.seg_base[I + 1] - a.seg_base[I];
            base = (long long)a.seg_base[I] * a.R + (o - I * a.R);
            stride = a.R;
        } else {
            K = a.NS;
            base = o;
            stride = a.n;
        }
        const T* __restrict__ p = a.part + base;
        acc = ordered_batch_sum<T, MERGE_BATCH>(acc, g, K, SPLIT,
                                                [&](int k) { return p + (long long)k * stride; });
    }
    part[g][lane] = acc;
    __syncthreads();
#pragma unroll
    for (int w = SPLIT / 2; w >= 1; w >>= 1) {
        if (g < w) part[g][lane] = E::add(part[g][lane], part[g + w][lane]);
        __syncthreads();
    }
    if (g == 0 && o < a.leny) {
        const T tot = part[0][lane];
        T* yp = a.y + a.ky + (long long)o * a.incy;
        T r = E::mul(a.alpha, tot);
        if (!a.beta_zero) r = E::add(r, E::mul(a.beta, *yp));
        *yp = r;
    }
}

}  // namespace xsymv
