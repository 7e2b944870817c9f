// xtrmv_strip.hpp -- triangular matrix-vector product x := op(T)*x on gfx950
// (T the stored triangle of A, column-major; op = T, T^T or T^H; unit or
// non-unit diagonal).
//
// Another of the Level-2 BLAS that the CUDA-xSYMV report's §5 carries its
// approach to: the triangle that SYMV reads once for two uses is here read
// once for one use, so the streaming machinery and the work split are SYMV's
// and the product moves the same bytes as SYMV at half the flops.
//
//  * Work split: the row-strip plan of the symmetric kernels.  Strip i (rows
//    [iR, iR+R)) holds exactly the columns with stored elements in its rows
//    (L: [0, min(n, iR+R)); U: [iR, n)), the strips' columns form one
//    sequence cut into pieces of equal cost over the resident workgroups.
//  * Per column the W waves of a workgroup read one contiguous run of R rows
//    with raw-buffer loads bounded above by the stored rows (L: row n; U: the
//    diagonal, included unless the diagonal is unit).  The L diagonal band
//    needs a lower bound as well: those groups take element loads, the offset
//    of an unstored row moved past the byte count (no access).
//  * 'N': output r needs the row role only -- each lane keeps SW*VEC row
//    partials for its whole segment and writes them once (no LDS, no barriers).
//  * 'T'/'C': output c needs the column role only -- per group of G columns a
//    halving lane exchange, then the waves added in wave order through LDS,
//    written to colpart[strip][column].
//  * trmv_merge adds the partials of each output in a fixed order (plus x_r
//    itself for a unit diagonal, whose stored value is never read) and writes
//    x; the streaming kernel has read all of x before the merge starts.
#pragma once

#include "xsymv_strip.hpp"

namespace xsymv {

template <class T>
struct TrmvArgs {
    const T* A;
    const T* x;           // contiguous copy of the input vector
    T* rowpart;           // 'N': [nseg][R]
    T* colpart;           // 'T', 'C': [NS][n]
    const StripBlock* blocks;
    const int* strip_base;  // [NS+1]
    long long lda;
    int n;
};

// TR: 0 'N', 1 'T', 2 'C'
template <class T, bool UPPER, int TR, bool UNIT, int W, int SW, int G, bool NT, int CBUF>
__global__ __launch_bounds__(64 * W) void trmv_strip(TrmvArgs<T> a)
{
    using E = Elem<T>;
    constexpr int V = E::VEC;
    constexpr int H = 64 * V;
    constexpr int RW = SW * H;  // rows per wave
    constexpr int R = W * RW;
    constexpr int ES = (int)sizeof(T);
    constexpr int GROUP = 64 / G;
    constexpr int DU = UNIT ? 1 : 0;  // the diagonal is outside the read triangle
    constexpr int FAR = 0x7fffff00;   // an offset past every byte count
    static_assert(CBUF % G == 0, "column buffer holds whole groups");

    __shared__ T colred[TR == 0 ? 1 : W][TR == 0 ? 1 : CBUF];

    const StripBlock bd = a.blocks[blockIdx.x];
    const int n = a.n;
    const long long lda = a.lda;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const T* __restrict__ A = a.A;
    const T* __restrict__ x = a.x;

    int u = bd.u0;
    int slot = bd.slot0;
    int strip = bd.strip0;
    while (u < bd.u1) {  // workgroup-uniform: one segment per iteration
        const int sb0 = a.strip_base[strip];
        const int useg = min(bd.u1, a.strip_base[strip + 1]);
        const int rs0 = strip * R;
        const int rs1 = min(n, rs0 + R);
        const int coff = (UPPER ? rs0 : 0) - sb0;  // column = sequence position + coff
        const int rw = rs0 + wave * RW;            // this wave's first row
        const bool wave_empty = rw >= rs1;

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
            // stored rows of column c: L [c + DU, n), U [0, c + 1 - DU)
            const bool empty = wave_empty || (UPPER ? (rw > jg + ng - 1 - DU)
                                                    : (rw + RW <= jg + DU));
            // L: some row of this wave lies above a column's first stored row
            const bool band = !UPPER && !empty && rw < jg + ng - 1 + DU;
            T cacc[G];
#pragma unroll
            for (int g = 0; g < G; ++g) cacc[g] = E::zero();
            if (empty) {
                // nothing stored in this wave's rows
            } else if (!band) {
                // FULL ('N'): every column of the group is real, so x needs no
                // select and is used by the multiply-adds only; compiled twice
                // where a lane's vector holds several elements.  For the fp32
                // types x at the column index is read by scalar loads (x is
                // the call's copy of the input, which no kernel writes).
                auto stream_group = [&](auto full) {
                    constexpr bool FULL = decltype(full)::value;
                    constexpr bool XS = E::SCALAR_X && TR == 0;
                    using cword = const __attribute__((address_space(4))) unsigned*;
                    T av[G][SW][V];
                    T xcol[G];
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const bool real = FULL || g < ng;
                        const int cc = real ? jg + g : jg;
                        // stored rows of this wave in column cc: [rw, bound)
                        const int bound = UPPER ? cc + 1 - DU : n;
                        const int rows = real ? min(RW, max(0, bound - rw)) : 0;
                        const auto rs = make_rsrc(A + (long long)cc * lda + rw, rows * ES);
#pragma unroll
                        for (int s = 0; s < SW; ++s)
                            E::template bload16<NT>(rs, (s * H + lane * V) * ES, av[g][s]);
                        if (TR == 0) {
                            const T xv = XS ? uniform_load<T>((cword)x, cc) : x[cc];
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
                if (TR == 0 && V > 1 && ng == G)
                    stream_group(std::integral_constant<bool, (TR == 0 && V > 1)>{});
                else
                    stream_group(std::false_type{});
            } else {
                // L diagonal band: element loads; rows above a column's first
                // stored row, or past n, read as zero without an access
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int col = jg + g;
                    const bool real = g < ng;
                    const int cc = real ? col : jg;  // jg is a real column
                    const auto rsr = make_rsrc(A + (long long)cc * lda + rw, real ? RW * ES : 0);
                    const T xcol = TR == 0 ? E::sel(real, x[cc], E::zero()) : E::zero();
#pragma unroll
                    for (int s = 0; s < SW; ++s)
#pragma unroll
                        for (int k = 0; k < V; ++k) {
                            const int r = rw + s * H + lane * V + k;
                            const bool st = r >= col + DU && r < n;
                            const T av = bload1<T>(rsr, st ? (s * H + lane * V + k) * ES : FAR);
                            if (TR == 0)
                                racc[s][k] = E::mac(racc[s][k], av, xcol);
                            else if (TR == 1)
                                cacc[g] = E::mac(cacc[g], av, xr[s][k]);
                            else
                                cacc[g] = E::macc(cacc[g], av, xr[s][k]);
                        }
                }
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

// Ordered merge: output o adds its terms in a fixed order -- 'N': the row
// partials of o's strip, segment by segment; 'T'/'C': the column partials of
// the strips that hold column o (L: strips I..NS-1, U: 0..I, I = o's strip)
// in ascending order -- then, for a unit diagonal, x_o itself.  SPLIT waves
// share 64 outputs (wave g takes the terms k with k % SPLIT == g) and meet in
// a fixed pairwise tree.  Each output reads its own input element before
// writing it, so x may be both the input copy and the output.
template <class T>
struct TrmvMergeArgs {
    const T* part;
    const int* seg_base;  // 'N': segments of strip i are [seg_base[i], seg_base[i+1])
    const T* xin;         // contiguous input vector (unit diagonal term)
    T* x;
    long long incx;
    long long kx;
    int n;
    int NS;
    int R;
    int upper;
    int trans;  // 0 'N', else 'T'/'C'
    int unit;
};

template <class T, int SPLIT>
__global__ __launch_bounds__(64 * SPLIT) void trmv_merge(TrmvMergeArgs<T> a)
{
    using E = Elem<T>;
    __shared__ T part[SPLIT][64];
    const int lane = threadIdx.x & 63;
    const int g = threadIdx.x >> 6;
    const int o = blockIdx.x * 64 + lane;
    T acc = E::zero();
    if (o < a.n) {
        const int I = o / a.R;
        long long base, stride;
        int K;
        if (a.trans == 0) {
            K = a.seg_base[I + 1] - a.seg_base[I];
            base = (long long)a.seg_base[I] * a.R + (o - I * a.R);
            stride = a.R;
        } else {
            const int c_lo = a.upper ? 0 : I;
            K = a.upper ? I + 1 : a.NS - I;
            base = (long long)c_lo * a.n + o;
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
    if (g == 0 && o < a.n) {
        T tot = part[0][lane];
        if (a.unit) tot = E::add(tot, a.xin[o]);
        a.x[a.kx + (long long)o * a.incx] = tot;
    }
}

}  // namespace xsymv
