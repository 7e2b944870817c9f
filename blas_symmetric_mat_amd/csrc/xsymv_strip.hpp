// xsymv_strip.hpp -- row-strip, evenly split kernels for y := alpha*S*x + beta*y
// on gfx950 (only one triangle of S stored, column-major).
//
// Each stored off-diagonal element is read once and used twice (its own row
// and, conjugated, the mirrored element's row), as in the CUDA-xSYMV report's
// algorithm (§2.1 Fig. 1); partial sums are combined in a fixed order, with no
// floating-point atomics, so results are bitwise identical from run to run
// (the report's aim, §2.1; it used an atomic ticket lock instead).
//
// Decomposition (gfx950-specific):
//  * Rows are cut into strips of R = W*SW*64*VEC rows.  Strip i stores, for
//    uplo = L, the columns [0, iR) in full plus the diagonal triangle of
//    columns [iR, iR+R); for U, the columns [iR+R, n) in full plus its
//    diagonal triangle.
//  * The strips' columns, concatenated in strip order, form one sequence.  It
//    is cut into G ranges of equal cost (stored elements), G = the number of
//    workgroups the GPU holds at once, so every workgroup streams the same
//    number of bytes and they all finish together.  A range may span strips;
//    its piece in one strip is a segment.
//  * A workgroup walks its columns in order.  For each column, wave w reads
//    its own SW stripes right below wave w-1's, so the workgroup reads one
//    contiguous run of R rows per column (long runs keep HBM efficient even
//    when the leading dimension is a power of two).
//  * Row role: each lane keeps SW*VEC row partials in registers for the whole
//    segment and writes them once to rowpart[segment][row].
//  * Column role: a column's sum over the strip's rows is finished inside the
//    workgroup (lane exchange per group of G columns, then the W waves added
//    in wave order through LDS) and written to colpart[strip][column].
//  * symv_strip_merge: y_r = beta*y_r + alpha*(sum of the row partials of r's
//    strip in segment order + sum of colpart[i][r] in strip order).
#pragma once

#include <hip/hip_ext.h>

#include <type_traits>

#include "xsymv_kernels.hpp"

namespace xsymv {

// Per workgroup: [u0, u1) in the column sequence, first segment slot, strip
// of u0, and that strip's entries of the plan's tables (where its sequence
// starts and ends, its first local column), so that a workgroup's first
// column loads depend on this one descriptor load alone.  32 bytes: read by
// one scalar load.
struct StripBlock {
    int u0;
    int u1;
    int slot0;
    int strip0;
    int sb0;   // strip_base[strip0]
    int sb1;   // strip_base[strip0 + 1]
    int col0;  // strip_col0[strip0] (a shard's product), else 0
    int pad;
};

template <class T>
struct StripArgs {
    const T* A;
    const T* x;           // contiguous
    T* rowpart;           // [nseg][R]
    T* colpart;           // [NS][n] (sharded: [NS][ncol])
    const StripBlock* blocks;
    const int* strip_base;  // [NS+1]: first sequence position of strip i
    long long lda;
    int n;
    // one shard's product only: A holds the shard's columns (local column l
    // is global column lcol[l], ascending)
    const int* lcol;        // [ncol]
    const int* gloc;        // [n]: local column of a global column, or -1
    const int* strip_col0;  // [NS]: first local column of strip i's sequence
    int ncol;
};

// Reads of A.  A wave's rows of column j are one run of SW*H elements
// starting at row rw.  Stored rows of column j: L: j < r < n (strictly below
// the diagonal), U: 0 <= r < j.  Both are "rows below an upper bound" once
// r > j is known, so whole groups are read with 16-byte raw-buffer loads whose
// byte count ends at that bound: rows at or past it read as zero without a
// memory access.  That covers the ragged last strip (L and U) and, for U, the
// diagonal band.  For L the band (rows around the diagonal) also needs a lower
// bound: a vector with no stored row is read at an offset past the byte count,
// and the one lane per column whose vector holds the diagonal row reads its 16
// bytes from the diagonal row instead (Hermitian: the row below it, plus the
// diagonal's real word on its own) and moves them to its rows, so no word
// outside the stored triangle is read.  The diagonal itself counts once, in
// the row role: for L inside the band, for U d_r * x_r is added at the end of
// the segment that holds column r.  For Hermitian products only the real word
// of a diagonal element is read.
//
// SHARD: one GPU's share of the product when the columns are dealt out in
// panels.  A is the shard's local matrix; the sequence runs over its local
// columns (those with stored rows in the strip form a contiguous range, as the
// local-to-global map ascends), addresses use the local column, triangle
// bounds and x the global one, and column partials are indexed locally.
// Element i of an array of T read through the constant address space by a
// wave-uniform index (scalar loads of its 32-bit words).
template <class T>
__device__ __forceinline__ T uniform_load(const __attribute__((address_space(4))) unsigned* p,
                                          int i)
{
    constexpr int NW = sizeof(T) / 4;
    unsigned w[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) w[k] = p[(long long)i * NW + k];
    T v;
    __builtin_memcpy(&v, w, sizeof(T));
    return v;
}

// The value of the diagonal element at byte offset `off` of a raw buffer: its
// first Elem<T>::DIAG_WORDS words (Hermitian: the real word; the imaginary
// word is not read), the others zero.  Past the byte count: zero, no access.
template <class T>
__device__ __forceinline__ T bload_diag(__amdgpu_buffer_rsrc_t r, int off)
{
    constexpr int NW = Elem<T>::DIAG_WORDS;
    unsigned w[sizeof(T) / 4] = {};
    if constexpr (NW == 1) {
        w[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    } else {
        static_assert(NW == 2, "one or two words");
        const unsigned long long d =
            __builtin_bit_cast(unsigned long long, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
        w[0] = (unsigned)d;
        w[1] = (unsigned)(d >> 32);
    }
    T v;
    __builtin_memcpy(&v, w, sizeof(T));
    return v;
}

template <class T, bool UPPER, int W, int SW, int G, bool NT, int CBUF, bool SHARD = false>
__global__ __launch_bounds__(64 * W) void symv_strip(StripArgs<T> a)
{
    using E = Elem<T>;
    constexpr int V = E::VEC;
    constexpr int H = 64 * V;
    constexpr int RW = SW * H;  // rows per wave
    constexpr int R = W * RW;
    constexpr int GROUP = 64 / G;
    constexpr int FAR = 0x7fffff00;  // an offset past every byte count
    static_assert(CBUF % G == 0, "column buffer holds whole groups");

    __shared__ T colred[W][CBUF];

    // the descriptor through the constant address space: one scalar load
    // of its 32 bytes
    using cblock = const __attribute__((address_space(4))) StripBlock*;
    const cblock bp = (cblock)a.blocks + blockIdx.x;
    const StripBlock bd{bp->u0, bp->u1, bp->slot0, bp->strip0, bp->sb0, bp->sb1, bp->col0, 0};
    const int n = a.n;
    const long long lda = a.lda;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const T* __restrict__ A = a.A;
    const T* __restrict__ x = a.x;
    // the column map is read at wave-uniform indices only: read it through
    // the constant address space (scalar loads), so that no vector load has
    // to complete before the element addresses that depend on it
    using cmap = const __attribute__((address_space(4))) int*;
    const cmap lcol = (cmap)a.lcol;
    // x at a column's index is wave-uniform too.  Read by scalar loads it
    // stays off the vector-memory counter, which retires in order, so that
    // using it does not wait for the column loads issued before it; measured,
    // that pays for the fp32 types with uplo = L only
    constexpr bool XS = E::SCALAR_X && !UPPER;
    using cword = const __attribute__((address_space(4))) unsigned*;
    const cword xw = (cword)a.x;
    const int* __restrict__ gloc = a.gloc;

    int u = bd.u0;
    int slot = bd.slot0;
    int strip = bd.strip0;
    // this strip's table entries: from the descriptor for the first segment,
    // from the tables for a later one
    int sb_lo = bd.sb0, sb_hi = bd.sb1, scol0 = bd.col0;
    while (u < bd.u1) {  // workgroup-uniform: one segment per iteration
        const int sb0 = sb_lo;
        const int useg = min(bd.u1, sb_hi);
        const int rs0 = strip * R;
        const int rs1 = min(n, rs0 + R);
        // (local) column = sequence position + coff
        const int coff = (UPPER ? (SHARD ? scol0 : rs0) : 0) - sb0;
        const int rw = rs0 + wave * RW;            // this wave's first row
        const bool wave_empty = rw >= rs1;

        T racc[SW][V];
        T xr[SW][V];
#pragma unroll
        for (int s = 0; s < SW; ++s)
#pragma unroll
            for (int k = 0; k < V; ++k) {
                racc[s][k] = E::zero();
                const int r = rw + s * H + lane * V + k;
                const T v = x[r < rs1 ? r : rs1 - 1];
                xr[s][k] = E::sel(r < rs1, v, E::zero());
            }
        // U: the diagonal of the rows whose column is in this segment (local
        // columns [c0, c1)), loaded now and added at the segment's end, so
        // that the end waits on no load (a segment of the diagonal triangle
        // holds several of them, each in its own cache line).  A shard's
        // segment may hold no column: a strip without any of its columns
        // that a workgroup's range steps through.
        constexpr int NDG = UPPER ? SW : 1;
        T dg[NDG][V];
        bool din[NDG][V];
        const bool has_diag = UPPER && (!SHARD || useg > u);
        if constexpr (UPPER) {
            const int c0 = u + coff, c1 = useg + coff;
#pragma unroll
            for (int s = 0; s < SW; ++s)
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const int r = rw + s * H + lane * V + k;
                    // the row's own column, locally (-1: another shard's)
                    const int lr = has_diag ? (SHARD ? gloc[r < rs1 ? r : rs1 - 1] : r) : -1;
                    const bool in = has_diag && lr >= c0 && lr < c1 && r < rs1;
                    // c0 < ncol is a real local column, its diagonal a stored
                    // element (no load at all when the segment holds none)
                    const long long cl = in ? lr : c0;
                    const long long rg = in ? r : (SHARD ? (has_diag ? lcol[c0] : 0) : c0);
                    din[s][k] = in;
                    dg[s][k] = has_diag ? E::diag_load(A + cl * lda + rg) : E::zero();
                }
        }

        int jbuf = u + coff;  // first column held in colred
        int nbuf = 0;         // columns held in colred
#pragma unroll 1
        for (int g0 = u; g0 < useg; g0 += G) {
            const int jg = g0 + coff;          // first column of the group
            const int ng = min(G, useg - g0);  // real columns in the group
            // global indices of the group's first and last columns
            const int gfirst = SHARD ? lcol[jg] : jg;
            const int glast = SHARD ? lcol[jg + ng - 1] : jg + ng - 1;
            // no stored element of the group in this wave's rows
            const bool empty =
                wave_empty || (UPPER ? (rw >= glast) : (rw + RW <= gfirst));
            // every real column of the group is left of this wave's rows (L)
            const bool band = !UPPER && !empty && rw < glast + 1;
            T cacc[G];
            // The group's loads and multiply-adds.  FULL: every column of the
            // group is real (all groups but a segment's last), so x is used by
            // the multiply-adds only; a select on it would make the compiler
            // wait for its load before issuing the next column loads.  Measured,
            // the second copy of the body pays where a lane's vector holds
            // several elements and costs the 16-byte types.
            auto stream_group = [&](auto full) {
                constexpr bool FULL = decltype(full)::value;
                if (!band) {
                    T av[G][SW][V];
                    T xcol[G];
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const bool real = FULL || g < ng;
                        const int cl = real ? jg + g : jg;      // local column
                        const int cc = SHARD ? lcol[cl] : cl;  // global column
                        // stored rows of this wave in column cc: [rw, bound)
                        const int bound = UPPER ? cc : n;
                        const int rows = real ? min(RW, max(0, bound - rw)) : 0;
                        const auto rs =
                            make_rsrc(A + (long long)cl * lda + rw, rows * (int)sizeof(T));
#pragma unroll
                        for (int s = 0; s < SW; ++s)
                            E::template bload16<NT>(rs, (s * H + lane * V) * (int)sizeof(T),
                                                    av[g][s]);
                        const T xv = XS ? uniform_load<T>(xw, cc) : x[cc];
                        xcol[g] = FULL ? xv : E::sel(real, xv, E::zero());
                    }
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        cacc[g] = E::zero();
#pragma unroll
                        for (int s = 0; s < SW; ++s)
#pragma unroll
                            for (int k = 0; k < V; ++k) {
                                racc[s][k] = E::mac(racc[s][k], av[g][s][k], xcol[g]);
                                cacc[g] = E::macc(cacc[g], av[g][s][k], xr[s][k]);
                            }
                    }
                } else {
                    // L diagonal band: as above, with a lower bound.  A vector
                    // with no stored row reads past the byte count (zeros, no
                    // access).  The lane whose vector holds the diagonal row
                    // reads the 16 bytes that start at the diagonal (Hermitian:
                    // one row below it, and the diagonal's real word by a load
                    // of its own) and shifts them to its rows with selects, so
                    // that nothing above the diagonal is read.  The diagonal
                    // counts in the row role only.
                    constexpr int DH = E::DIAG_WORDS * 4 < (int)sizeof(T);  // Hermitian
                    T av[G][SW][V];
                    T dv[G][SW];  // Hermitian: the diagonal, in the lane that holds it
                    T xcol[G];
                    int cg[G];
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const bool real = FULL || g < ng;
                        const int cl = real ? jg + g : jg;      // local column
                        const int cc = SHARD ? lcol[cl] : cl;  // global column
                        const int rows = real ? min(RW, max(0, n - rw)) : 0;
                        const auto rs =
                            make_rsrc(A + (long long)cl * lda + rw, rows * (int)sizeof(T));
#pragma unroll
                        for (int s = 0; s < SW; ++s) {
                            const int rf = rw + s * H + lane * V;   // the vector's first row
                            const int r0 = rf > cc ? rf : cc + DH;  // first row it reads
                            E::template bload16<NT>(
                                rs, r0 < rf + V ? (r0 - rw) * (int)sizeof(T) : FAR, av[g][s]);
                            if constexpr (DH)
                                dv[g][s] = bload_diag<T>(
                                    rs, rf <= cc && cc < rf + V ? (cc - rw) * (int)sizeof(T) : FAR);
                        }
                        const T xv = XS ? uniform_load<T>(xw, cc) : x[cc];
                        xcol[g] = FULL ? xv : E::sel(real, xv, E::zero());
                        cg[g] = real ? cc : -1;
                    }
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        cacc[g] = E::zero();
#pragma unroll
                        for (int s = 0; s < SW; ++s) {
                            const int rf = rw + s * H + lane * V;
                            // rows the loaded vector starts below this lane's
                            // first row (0 except in the lane with the diagonal)
                            const int sh = rf > cg[g] ? 0 : cg[g] + DH - rf;
#pragma unroll
                            for (int k = 0; k < V; ++k) {
                                // row rf + k is element k - sh of the loaded vector
                                T v = av[g][s][k];
                                if constexpr (V > 1) {
                                    v = E::sel(sh == 0, v, E::zero());
#pragma unroll
                                    for (int j = 0; j < k; ++j)
                                        v = E::sel(sh == k - j, av[g][s][j], v);
                                }
                                const bool dg = rf + k == cg[g];
                                T ac, ar;  // column role (off-diagonal only), row role
                                if constexpr (DH) {
                                    ac = v;
                                    ar = E::sel(dg, dv[g][s], v);
                                } else {
                                    ac = E::sel(dg, E::zero(), v);
                                    ar = v;
                                }
                                racc[s][k] = E::mac(racc[s][k], ar, xcol[g]);
                                cacc[g] = E::macc(cacc[g], ac, xr[s][k]);
                            }
                        }
                    }
                }
            };
            if (empty) {
#pragma unroll
                for (int g = 0; g < G; ++g) cacc[g] = E::zero();
            } else if (V > 1 && ng == G) {
                stream_group(std::integral_constant<bool, (V > 1)>{});
            } else {
                stream_group(std::false_type{});
            }
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
                    a.colpart[(long long)strip * (SHARD ? a.ncol : n) + jbuf + c] = sum;
                }
                __syncthreads();
                jbuf += nreal;
                nbuf = 0;
            }
        }
        if constexpr (UPPER) {
            if (has_diag) {
#pragma unroll
                for (int s = 0; s < SW; ++s)
#pragma unroll
                    for (int k = 0; k < V; ++k)
                        racc[s][k] = E::mac(racc[s][k], E::sel(din[s][k], dg[s][k], E::zero()),
                                            xr[s][k]);
            }
        }
        // this wave's row partials for the segment
        T* __restrict__ rp = a.rowpart + (long long)slot * R;
#pragma unroll
        for (int s = 0; s < SW; ++s)
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const int r = rw + s * H + lane * V + k;
                if (r < rs1) rp[r - rs0] = racc[s][k];
            }
        u = useg;
        ++slot;
        ++strip;
        if (u < bd.u1) {  // another strip follows (strip < NS)
            sb_lo = sb_hi;
            sb_hi = a.strip_base[strip + 1];
            if constexpr (SHARD && UPPER) scol0 = a.strip_col0[strip];
        }
    }
}

// Ordered merge for the strip decomposition: row r of strip I adds its row
// partials slot by slot (segments of strip I in order), then the column
// partials colpart[i][r] of the strips that hold column r (L: i >= I,
// U: i <= I) in ascending i.  A workgroup of SPLIT waves takes ROWS
// consecutive rows (64 or 32); the 64 / ROWS lane groups of a wave and the
// waves give SPLIT * 64 / ROWS streams, stream v taking the terms k with
// k % streams == v; the subtotals meet in a fixed pairwise tree.  ROWS = 32
// runs twice as many workgroups, for orders whose 64-row blocks would leave
// CUs idle.
constexpr int MERGE_SEG_INLINE = 64;

template <class T>
struct StripMergeArgs {
    const T* rowpart;
    const T* colpart;
    const int* seg_base;  // [NS+1]: segments of strip i are [seg_base[i], seg_base[i+1])
    T* y;
    long long incy;
    long long ky;
    T alpha;
    T beta;
    int n;
    int NS;
    int R;
    int upper;
    int beta_zero;
    const int* gloc;  // sharded product only
    int ncol;
    // seg_base itself (NS + 1 entries) when it fits: the kernel arguments
    // come with the first scalar load, so the partials' addresses wait on no
    // table in memory
    int seg_inline[MERGE_SEG_INLINE];
};

// SHARD: the shard's partial vector -- column partials only for the rows
// whose column the shard owns (local index gloc[i], rows of ncol), no alpha or
// beta: y is the contiguous partial p.  INL: seg_base from the arguments.
template <class T, int SPLIT, bool SHARD = false, int ROWS = 64, bool INL = false>
__global__ __launch_bounds__(64 * SPLIT) void symv_strip_merge(StripMergeArgs<T> a)
{
    using E = Elem<T>;
    constexpr int GROUPS = 64 / ROWS;      // lane groups per wave
    constexpr int V = SPLIT * GROUPS;      // streams
    static_assert(ROWS == 64 || ROWS == 32, "64 or 32 rows per workgroup");
    __shared__ T part[V][ROWS];
    const int lane = threadIdx.x & 63;
    const int v = (threadIdx.x >> 6) * GROUPS + lane / ROWS;  // this lane's stream
    const int rl = lane % ROWS;
    const int i = blockIdx.x * ROWS + rl;
    // the workgroup's rows lie in one strip (R is a multiple of ROWS): its
    // segment range is read by scalar loads, and y_i (when beta != 0) is
    // loaded now, so that neither waits at the end
    const int I = (int)((blockIdx.x * (unsigned)ROWS) / (unsigned)a.R);  // below n: 32 bits
    using cint = const __attribute__((address_space(4))) int*;
    const int s_lo = INL ? a.seg_inline[I] : ((cint)a.seg_base)[I];
    const int nrow = (INL ? a.seg_inline[I + 1] : ((cint)a.seg_base)[I + 1]) - s_lo;
    T* yp = nullptr;
    T yv = E::zero();
    if constexpr (!SHARD) {
        yp = a.y + a.ky + (long long)i * a.incy;
        if (v == 0 && i < a.n && !a.beta_zero) yv = *yp;
    }
    T acc = E::zero();
    if (i < a.n) {
        const int c_lo = a.upper ? 0 : I;
        const int li = SHARD ? a.gloc[i] : i;  // the row's column, locally
        const int ncol = li < 0 ? 0 : (a.upper ? I + 1 : a.NS - I);
        const int ntot = nrow + ncol;
        const long long cstride = SHARD ? a.ncol : a.n;
        const T* __restrict__ rp = a.rowpart + (long long)s_lo * a.R + (i - I * a.R);
        const T* __restrict__ cp = a.colpart + (long long)c_lo * cstride + li;
        acc = ordered_batch_sum<T, MERGE_BATCH>(acc, v, ntot, V, [&](int k) {
            return k < nrow ? rp + (long long)k * a.R : cp + (long long)(k - nrow) * cstride;
        });
    }
    part[v][rl] = acc;
    __syncthreads();
#pragma unroll
    for (int w = V / 2; w >= 1; w >>= 1) {
        if (v < w) part[v][rl] = E::add(part[v][rl], part[v + w][rl]);
        __syncthreads();
    }
    if (v == 0 && i < a.n) {
        const T tot = part[0][rl];
        if constexpr (SHARD) {
            a.y[i] = tot;
        } else {
            T r = E::mul(a.alpha, tot);
            if (!a.beta_zero) r = E::add(r, E::mul(a.beta, yv));
            *yp = r;
        }
    }
}

// Rows per merge workgroup for order n: 32 below 16384 (twice the
// workgroups), else 64.
constexpr int MERGE_ROWS_SMALL_BELOW = 16384;

// Launches the merge for order n; `stop` (timing only) takes the merge's own
// end time from its dispatch.  h_seg (host copy of seg_base, NS + 1 entries)
// given and short enough: the table goes in the arguments.  Returns the
// launch's error.
template <class T, int SPLIT, bool SHARD = false>
hipError_t launch_strip_merge(StripMergeArgs<T> ma, int n, hipStream_t stream,
                              hipEvent_t stop = nullptr, const int* h_seg = nullptr)
{
    const bool small = n < MERGE_ROWS_SMALL_BELOW;
    const bool inl = h_seg != nullptr && ma.NS + 1 <= MERGE_SEG_INLINE;
    if (inl) {
        for (int i = 0; i <= ma.NS; ++i) ma.seg_inline[i] = h_seg[i];
    }
    auto k = small ? (inl ? &symv_strip_merge<T, SPLIT, SHARD, 32, true>
                          : &symv_strip_merge<T, SPLIT, SHARD, 32, false>)
                   : (inl ? &symv_strip_merge<T, SPLIT, SHARD, 64, true>
                          : &symv_strip_merge<T, SPLIT, SHARD, 64, false>);
    const int rows = small ? 32 : 64;
    const dim3 grid((n + rows - 1) / rows), block(64 * SPLIT);
    if (stop == nullptr) {
        k<<<grid, block, 0, stream>>>(ma);
        return hipGetLastError();
    }
    void* p[] = {&ma};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(k), grid, block, p, 0, stream, nullptr,
                              stop, 0);
}

// Rank-ordered combination of the shards' partials: y_i := beta*y_i +
// alpha*(P[0][i] + P[1][i] + ...), summed from shard 0 up (beta = 0: y not
// read).  One lane per output; the partials' reads are coalesced.
template <class T>
struct CombineArgs {
    const T* P;
    T* y;
    long long ldp;
    long long incy;
    long long ky;
    T alpha;
    T beta;
    int n;
    int nshards;
    int beta_zero;
};

template <class T>
__global__ __launch_bounds__(256) void symv_combine(CombineArgs<T> a)
{
    using E = Elem<T>;
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= a.n) return;
    // the partials are loaded 8 at a time (all in flight together) and added
    // in rank order
    T sum = a.P[i];
    for (int g0 = 1; g0 < a.nshards; g0 += 8) {
        T v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            v[k] = g0 + k < a.nshards ? a.P[(long long)(g0 + k) * a.ldp + i] : E::zero();
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (g0 + k < a.nshards) sum = E::add(sum, v[k]);
    }
    T* yp = a.y + a.ky + (long long)i * a.incy;
    T r = E::mul(a.alpha, sum);
    if (!a.beta_zero) r = E::add(E::mul(a.beta, *yp), r);
    *yp = r;
}

}  // namespace xsymv
