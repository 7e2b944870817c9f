// xsymv_kernels.hpp -- gfx950 kernels for y := alpha*S*x + beta*y, where S is
// symmetric (or Hermitian) and only one triangle of it is stored, column-major.
//
// Method (the CUDA-xSYMV report, §2.1 Fig. 1 and §2.1 Fig. 3): every stored
// off-diagonal element a = A(i,j) is read from memory once and used twice,
// once for its own row (y_i += a*x_j) and once for the mirrored element
// (y_j += conj(a)*x_i); the diagonal contributes once; partial sums produced
// by different workgroups are combined in a fixed order, so that results are
// bitwise identical from run to run (the report's stated aim, reached there
// with an atomic ticket lock; here with a workspace and an ordered merge).
//
// Decomposition used here (gfx950-specific, not the report's):
//  * The stored triangle is cut into column panels of NB = W*CW columns.
//    Panel p owns columns [p*NB, p*NB+NB).  Its stored rows are split into a
//    diagonal tile (the NB x NB block on the diagonal) and off-diagonal tiles
//    of up to R = S*H rows.  One workgroup processes one tile.
//  * Workgroup = W wave64s.  Wave w owns CW consecutive columns of the panel;
//    lane l owns VEC consecutive rows in each of the S stripes of H = 64*VEC
//    rows, so one 16-byte load per lane covers 64*VEC contiguous rows of one
//    column (fully coalesced, column-major).
//  * Row role: each lane accumulates its rows over its wave's columns in
//    registers; the W waves' partials are added in LDS in wave order and the
//    tile writes one partial per row to rowpart[p][row].
//  * Column role: each lane accumulates its column sums over all stripes in
//    registers; a fixed butterfly across the 64 lanes finishes them and the
//    tile writes NB column partials to colpart[slot][*].
//  * symv_merge then forms y_i = beta*y_i + alpha*(sum of row partials of
//    row i in panel order + sum of column partials of column i in tile order).
// Nothing is added with atomics, and the order of every addition depends only
// on n, uplo and the tile shape, never on scheduling.
#pragma once

#include "xsymv_arith.hpp"

namespace xsymv {

// One workgroup's tile.  rows [r0, r1), panel p, colpart slot, kind.
struct TileDesc {
    int p;
    int r0;
    int r1;
    int slot_flags;  // slot << 2 | kind
};
// Tile kinds: full (R rows, NB columns, strictly off the diagonal), the
// diagonal block of a panel, or ragged (fewer rows or columns than the shape).
enum : int { TILE_FULL = 0, TILE_DIAG = 1, TILE_RAGGED = 2 };

template <class T>
struct SymvArgs {
    const T* A;
    const T* x;        // contiguous (gathered beforehand for incx != 1)
    T* rowpart;        // [P][n]
    T* colpart;        // [nslots][NB]
    const TileDesc* tiles;
    long long lda;
    int n;
};

// ---------------------------------------------------------------------------
// Column sums across the 64 lanes of a wave: CW values per lane in, each
// lane with (lane & (64/CW - 1)) == 0 ends holding the full sum of value
// index idx(lane).  Halving exchange: at each step a lane gives away half of
// its values to its partner and adds the partner's half of the other values,
// so the work is CW-1 additions instead of 6*CW.  The order is fixed.
template <class T, int CW>
__device__ __forceinline__ void wave_transpose_reduce(T (&v)[CW], int lane)
{
    using E = Elem<T>;
    int cnt = CW;
    int m = 32;
#pragma unroll
    for (int step = 0; step < 6; ++step) {
        if (cnt > 1) {
            const int half = cnt >> 1;
            const bool up = (lane & m) != 0;
#pragma unroll
            for (int i = 0; i < CW / 2; ++i) {
                if (i < half) {
                    const T give = E::sel(up, v[i], v[i + half]);
                    const T keep = E::sel(up, v[i + half], v[i]);
                    const T got = E::shfl_xor(give, m);
                    // (lower lane's value) + (upper lane's value) on both sides
                    v[i] = E::add(E::sel(up, got, keep), E::sel(up, keep, got));
                }
            }
            cnt = half;
        } else {
            const T got = E::shfl_xor(v[0], m);
            const bool up = (lane & m) != 0;
            v[0] = E::add(E::sel(up, got, v[0]), E::sel(up, v[0], got));
        }
        m >>= 1;
    }
}

// Index of the column sum a lane holds after wave_transpose_reduce.
template <int CW>
__device__ __forceinline__ int wave_transpose_index(int lane)
{
    int idx = 0;
    int cnt = CW;
    int m = 32;
    int base = 0;
#pragma unroll
    for (int step = 0; step < 6; ++step) {
        if (cnt > 1) {
            const int half = cnt >> 1;
            if (lane & m) base += half;
            cnt = half;
        }
        m >>= 1;
    }
    idx = base;
    return idx;
}

// ---------------------------------------------------------------------------
// Element (r, col) of a diagonal or ragged tile, branch-free so that every
// load of a column can be in flight at once.  `cc` is a valid column (col
// itself when col < n); an element outside the stored triangle or outside
// [.., r1) is not loaded: the lane loads the stored diagonal element (cc, cc)
// instead and the value is discarded by a select (never by a multiply, so
// NaN or Inf there cannot leak).  The diagonal element of a Hermitian matrix
// is its real part.  Returns the value for the row role; *off is the value
// for the column role (zero on the diagonal, which counts once).
template <class T, bool UPPER>
__device__ __forceinline__ T masked_elem(const T* __restrict__ Acc, int r, int r1, int col,
                                         int cc, bool colok, bool diag, T* off)
{
    using E = Elem<T>;
    const bool in = colok && r < r1 && (!diag || (UPPER ? (r <= col) : (r >= col)));
    const bool dg = diag && (r == col);
    const T v = E::load_any(Acc + (in ? r : cc), dg || !in);
    const T a = E::sel(in, v, E::zero());
    *off = E::sel(dg, E::zero(), a);
    return a;
}

// ---------------------------------------------------------------------------
// Main streaming kernel.  Template parameters:
//   T      element type; UPPER: stored triangle
//   W      waves per workgroup; CW columns per wave (NB = W*CW)
//   S      stripes of H = 64*VEC rows per tile (R = S*H): each wave reads
//          every one of its columns as one contiguous run of R rows
//   NT     non-temporal loads for A (streamed once)
//   XLDS   keep the tile's x rows in LDS (one 16-byte LDS read per 16-byte
//          load of A) instead of registers, so that long runs (large S) do
//          not cost occupancy
// Every load of A is issued without a data-dependent branch, so the compiler
// can keep many 16-byte loads in flight per wave.  Elements outside the
// stored triangle are never loaded: predicated-off lanes load a stored
// element instead (the diagonal of a valid column) and discard it.
template <class T, bool UPPER, int W, int CW, int S, bool NT, bool XLDS>
__global__ __launch_bounds__(64 * W) void symv_tiles(SymvArgs<T> args)
{
    using E = Elem<T>;
    constexpr int V = E::VEC;
    constexpr int H = 64 * V;
    constexpr int R = S * H;
    constexpr int NB = W * CW;

    // x rows of the tile while streaming (XLDS), then the waves' row partials
    __shared__ T red[W][R];

    const TileDesc d = args.tiles[blockIdx.x];
    const int p = d.p;
    const int r0 = d.r0;
    const int r1 = d.r1;
    const int slot = d.slot_flags >> 2;
    const int kind = d.slot_flags & 3;
    const int n = args.n;
    const long long lda = args.lda;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c0 = p * NB;
    const int cw0 = c0 + wave * CW;  // first column of this wave
    const T* __restrict__ A = args.A;
    const T* __restrict__ x = args.x;

    T racc[S][V];
    T cacc[CW];
    T xreg[XLDS ? 1 : S][V];
    T xc[CW];
#pragma unroll
    for (int c = 0; c < CW; ++c) {
        cacc[c] = E::zero();
        const int col = cw0 + c;
        const T v = x[col < n ? col : n - 1];
        xc[c] = E::sel(col < n, v, E::zero());
    }
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int k = 0; k < V; ++k) racc[s][k] = E::zero();
    if constexpr (XLDS) {
        T* xs = &red[0][0];
        for (int i = threadIdx.x; i < R; i += 64 * W) {
            const int r = r0 + i;
            const T v = x[r < r1 ? r : r1 - 1];
            xs[i] = E::sel(r < r1, v, E::zero());
        }
        __syncthreads();
    } else {
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const int r = r0 + s * H + lane * V + k;
                const T v = x[r < r1 ? r : r1 - 1];
                xreg[XLDS ? 0 : s][k] = E::sel(r < r1, v, E::zero());
            }
    }
    // x at the rows of stripe s for this lane
    auto xrow = [&](int s, T (&xv)[V]) {
        if constexpr (XLDS) {
            const T* xs = &red[0][0] + s * H + lane * V;
#pragma unroll
            for (int k = 0; k < V; ++k) xv[k] = xs[k];
        } else {
#pragma unroll
            for (int k = 0; k < V; ++k) xv[k] = xreg[XLDS ? 0 : s][k];
        }
    };

    if (kind == TILE_FULL) {
        // R rows, all NB columns stored, strictly off the diagonal.
        const T* __restrict__ Ab = A + (long long)cw0 * lda + r0 + lane * V;
#pragma unroll
        for (int c = 0; c < CW; ++c) {
#pragma unroll
            for (int s = 0; s < S; ++s) {
                T a[V], xv[V];
                E::template load16<NT>(Ab + c * lda + s * H, a);
                xrow(s, xv);
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    racc[s][k] = E::mac(racc[s][k], a[k], xc[c]);
                    cacc[c] = E::macc(cacc[c], a[k], xv[k]);
                }
            }
        }
    } else {
        // Diagonal block or ragged tile (fewer rows, or columns past n):
        // element loads at clamped addresses, all issued without branches.
        const bool diag = (kind == TILE_DIAG);
#pragma unroll
        for (int c = 0; c < CW; ++c) {
            const int col = cw0 + c;
            const bool colok = col < n;
            const int cc = colok ? col : c0;  // c0 < n always
            const T* __restrict__ Acc = A + (long long)cc * lda;
#pragma unroll
            for (int s = 0; s < S; ++s) {
                T xv[V];
                xrow(s, xv);
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    T off;
                    const T a = masked_elem<T, UPPER>(Acc, r0 + s * H + lane * V + k, r1, col,
                                                      cc, colok, diag, &off);
                    racc[s][k] = E::mac(racc[s][k], a, xc[c]);
                    cacc[c] = E::macc(cacc[c], off, xv[k]);
                }
            }
        }
    }

    // Column role: finish the sums across lanes, write NB partials.
    wave_transpose_reduce<T, CW>(cacc, lane);
    {
        constexpr int GROUP = 64 / CW;  // lanes sharing one finished sum
        if ((lane & (GROUP - 1)) == 0) {
            const int idx = wave_transpose_index<CW>(lane);
            args.colpart[(long long)slot * NB + wave * CW + idx] = cacc[0];
        }
    }

    // Row role: add the W waves' partials in wave order through LDS.
    if constexpr (XLDS) __syncthreads();  // every wave is done with the x rows
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int k = 0; k < V; ++k)
            red[wave][s * H + lane * V + k] = racc[s][k];
    __syncthreads();
    T* __restrict__ rp = args.rowpart + (long long)p * n;
    for (int i = threadIdx.x; i < R; i += 64 * W) {
        const int r = r0 + i;
        if (r < r1) {
            T sum = red[0][i];
#pragma unroll
            for (int w = 1; w < W; ++w) sum = E::add(sum, red[w][i]);
            rp[r] = sum;
        }
    }
}

// ---------------------------------------------------------------------------
// One lane's share of a merge: acc + t(k0) + t(k0 + step) + ... over k < kend,
// added in that order.  The terms are loaded NB at a time, all NB issued
// before the first is added, so a lane whose share is at most NB terms waits
// for one memory round trip (a loop that loads and adds term by term waits
// once per term).  Indices past kend load the batch's first term again (an
// address already in use, no branch) and are not added.  addr(k) is the
// address of term k.
template <class T, int NB, class Addr>
__device__ __forceinline__ T ordered_batch_sum(T acc, int k0, int kend, int step, Addr addr)
{
    using E = Elem<T>;
    for (int kb = k0; kb < kend; kb += NB * step) {
        T t[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int k = kb + b * step;
            t[b] = *addr(k < kend ? k : kb);
        }
        // keep the scheduler from moving each load down to its addition
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (kb + b * step < kend) acc = E::add(acc, t[b]);
    }
    return acc;
}

// Terms per batch of the merges' ordered sums.
constexpr int MERGE_BATCH = 8;

// ---------------------------------------------------------------------------
// Column-run kernel: the same tiles and partials as symv_tiles, organised so
// that registers do not grow with the panel width.  Each wave walks its CW
// columns one at a time; a column's R tile rows are one contiguous run of S
// 16-byte loads per lane, and the next column's run is loaded while the
// current one is used.  The tile's x rows sit in LDS.  A column's sum
// (column role) is finished right away by a fixed 64-lane butterfly, so the
// only long-lived accumulators are the S*VEC row partials.
template <class T>
__device__ __forceinline__ T wave_sum(T v, int lane)
{
    using E = Elem<T>;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const T got = E::shfl_xor(v, m);
        const bool up = (lane & m) != 0;
        v = E::add(E::sel(up, got, v), E::sel(up, v, got));
    }
    return v;
}

template <class T, bool UPPER, int W, int CW, int S, bool NT, bool PF>
__global__ __launch_bounds__(64 * W) void symv_runs(SymvArgs<T> args)
{
    using E = Elem<T>;
    constexpr int V = E::VEC;
    constexpr int H = 64 * V;
    constexpr int R = S * H;
    constexpr int NB = W * CW;

    // x rows of the tile while streaming, then the waves' row partials
    __shared__ T red[W][R];

    const TileDesc d = args.tiles[blockIdx.x];
    const int p = d.p;
    const int r0 = d.r0;
    const int r1 = d.r1;
    const int slot = d.slot_flags >> 2;
    const int kind = d.slot_flags & 3;
    const int n = args.n;
    const long long lda = args.lda;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c0 = p * NB;
    const int cw0 = c0 + wave * CW;  // first column of this wave
    const T* __restrict__ A = args.A;
    const T* __restrict__ x = args.x;
    T* __restrict__ colout = args.colpart + (long long)slot * NB + wave * CW;

    T racc[S][V];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int k = 0; k < V; ++k) racc[s][k] = E::zero();
    {
        T* xs = &red[0][0];
        for (int i = threadIdx.x; i < R; i += 64 * W) {
            const int r = r0 + i;
            const T v = x[r < r1 ? r : r1 - 1];
            xs[i] = E::sel(r < r1, v, E::zero());
        }
        __syncthreads();
    }
    const T* xs_lane = &red[0][0] + lane * V;

    if (kind == TILE_FULL) {
        // R rows, all NB columns stored, strictly off the diagonal.
        const T* __restrict__ Ab = A + (long long)cw0 * lda + r0 + lane * V;
        T cur[S][V];
        T xcol = x[cw0];
        if constexpr (PF) {
#pragma unroll
            for (int s = 0; s < S; ++s) E::template load16<NT>(Ab + s * H, cur[s]);
        }
#pragma unroll 1
        for (int c = 0; c < CW; ++c) {
            T nxt[PF ? S : 1][V];
            const int cn = (c + 1 < CW) ? c + 1 : c;  // wave-uniform
            if constexpr (PF) {
                const T* __restrict__ An = Ab + (long long)cn * lda;
#pragma unroll
                for (int s = 0; s < S; ++s) E::template load16<NT>(An + s * H, nxt[s]);
            } else {
                const T* __restrict__ Ac = Ab + (long long)c * lda;
#pragma unroll
                for (int s = 0; s < S; ++s) E::template load16<NT>(Ac + s * H, cur[s]);
            }
            const T xnext = x[cw0 + cn];
            T csum = E::zero();
            // x is re-read from LDS for every column: an opaque offset keeps
            // the compiler from hoisting it into S*VEC registers for the loop
            int xoff = 0;
            asm volatile("" : "+v"(xoff));
#pragma unroll
            for (int s = 0; s < S; ++s) {
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    racc[s][k] = E::mac(racc[s][k], cur[s][k], xcol);
                    csum = E::macc(csum, cur[s][k], xs_lane[xoff + s * H + k]);
                }
            }
            csum = wave_sum(csum, lane);
            if (lane == 0) colout[c] = csum;
            if constexpr (PF) {
#pragma unroll
                for (int s = 0; s < S; ++s)
#pragma unroll
                    for (int k = 0; k < V; ++k) cur[s][k] = nxt[PF ? s : 0][k];
            }
            xcol = xnext;
        }
    } else {
        // Diagonal block or ragged tile: element loads at clamped addresses,
        // all issued without branches.
        const bool diag = (kind == TILE_DIAG);
#pragma unroll 1
        for (int c = 0; c < CW; ++c) {
            const int col = cw0 + c;
            const bool colok = col < n;
            const int cc = colok ? col : c0;
            const T* __restrict__ Acc = A + (long long)cc * lda;
            const T xcol = E::sel(colok, x[cc], E::zero());
            T csum = E::zero();
#pragma unroll
            for (int s = 0; s < S; ++s) {
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    T off;
                    const T a = masked_elem<T, UPPER>(Acc, r0 + s * H + lane * V + k, r1, col,
                                                      cc, colok, diag, &off);
                    racc[s][k] = E::mac(racc[s][k], a, xcol);
                    csum = E::macc(csum, off, xs_lane[s * H + k]);
                }
            }
            csum = wave_sum(csum, lane);
            if (lane == 0) colout[c] = csum;
        }
    }

    // Row role: add the W waves' partials in wave order through LDS.
    __syncthreads();  // every wave is done with the x rows
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int k = 0; k < V; ++k)
            red[wave][s * H + lane * V + k] = racc[s][k];
    __syncthreads();
    T* __restrict__ rp = args.rowpart + (long long)p * n;
    for (int i = threadIdx.x; i < R; i += 64 * W) {
        const int r = r0 + i;
        if (r < r1) {
            T sum = red[0][i];
#pragma unroll
            for (int w = 1; w < W; ++w) sum = E::add(sum, red[w][i]);
            rp[r] = sum;
        }
    }
}

// ---------------------------------------------------------------------------
// Block-run kernel.  The W waves of a block walk the tile's NB columns
// together, one column (group) at a time; for each column, wave w reads its
// own SW stripes (SW*H rows) right below wave w-1's, so the block as a whole
// reads one contiguous run of W*SW*H rows per column.  Consequences:
//  * a wave owns its rows for the whole tile, so its row partials stay in
//    SW*VEC registers and are written straight to rowpart (no cross-wave
//    row reduction);
//  * column sums are finished per group of G consecutive columns by a fixed
//    lane exchange (wave_transpose_reduce), parked in LDS per wave, and added
//    across the W waves in wave order at the end of the tile.
// Tile shape: NB columns x R = W*SW*H rows.
template <class T, bool UPPER, int W, int NB, int SW, int G, bool NT>
__global__ __launch_bounds__(64 * W) void symv_block(SymvArgs<T> args)
{
    using E = Elem<T>;
    constexpr int V = E::VEC;
    constexpr int H = 64 * V;
    static_assert(NB % G == 0, "column groups must tile the panel");

    __shared__ T colred[W][NB];

    const TileDesc d = args.tiles[blockIdx.x];
    const int p = d.p;
    const int r0 = d.r0;
    const int r1 = d.r1;
    const int slot = d.slot_flags >> 2;
    const int kind = d.slot_flags & 3;
    const int n = args.n;
    const long long lda = args.lda;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c0 = p * NB;
    const int rw = r0 + wave * SW * H;  // first row of this wave
    const T* __restrict__ A = args.A;
    const T* __restrict__ x = args.x;

    T racc[SW][V];
    T xr[SW][V];
#pragma unroll
    for (int s = 0; s < SW; ++s)
#pragma unroll
        for (int k = 0; k < V; ++k) {
            racc[s][k] = E::zero();
            const int r = rw + s * H + lane * V + k;
            const T v = x[r < r1 ? r : r1 - 1];
            xr[s][k] = E::sel(r < r1, v, E::zero());
        }

    if (kind == TILE_FULL) {
        const T* __restrict__ Ab = A + (long long)c0 * lda + rw + lane * V;
#pragma unroll 1
        for (int cg = 0; cg < NB; cg += G) {
            T cacc[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int c = cg + g;
                T a[SW][V];
#pragma unroll
                for (int s = 0; s < SW; ++s)
                    E::template load16<NT>(Ab + (long long)c * lda + s * H, a[s]);
                const T xcol = x[c0 + c];
                cacc[g] = E::zero();
#pragma unroll
                for (int s = 0; s < SW; ++s)
#pragma unroll
                    for (int k = 0; k < V; ++k) {
                        racc[s][k] = E::mac(racc[s][k], a[s][k], xcol);
                        cacc[g] = E::macc(cacc[g], a[s][k], xr[s][k]);
                    }
            }
            wave_transpose_reduce<T, G>(cacc, lane);
            constexpr int GROUP = 64 / G;
            if ((lane & (GROUP - 1)) == 0)
                colred[wave][cg + wave_transpose_index<G>(lane)] = cacc[0];
        }
    } else {
        // Diagonal block or ragged tile: element loads at clamped addresses,
        // all issued without branches.
        const bool diag = (kind == TILE_DIAG);
#pragma unroll 1
        for (int cg = 0; cg < NB; cg += G) {
            T cacc[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int col = c0 + cg + g;
                const bool colok = col < n;
                const int cc = colok ? col : c0;
                const T* __restrict__ Acc = A + (long long)cc * lda;
                const T xcol = E::sel(colok, x[cc], E::zero());
                cacc[g] = E::zero();
#pragma unroll
                for (int s = 0; s < SW; ++s) {
#pragma unroll
                    for (int k = 0; k < V; ++k) {
                        T off;
                        const T a = masked_elem<T, UPPER>(Acc, rw + s * H + lane * V + k, r1,
                                                          col, cc, colok, diag, &off);
                        racc[s][k] = E::mac(racc[s][k], a, xcol);
                        cacc[g] = E::macc(cacc[g], off, xr[s][k]);
                    }
                }
            }
            wave_transpose_reduce<T, G>(cacc, lane);
            constexpr int GROUP = 64 / G;
            if ((lane & (GROUP - 1)) == 0)
                colred[wave][cg + wave_transpose_index<G>(lane)] = cacc[0];
        }
    }

    // Row role: this wave's rows are complete.
    T* __restrict__ rp = args.rowpart + (long long)p * n;
#pragma unroll
    for (int s = 0; s < SW; ++s)
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const int r = rw + s * H + lane * V + k;
            if (r < r1) rp[r] = racc[s][k];
        }
    // Column role: add the waves' sums in wave order.
    __syncthreads();
    for (int c = threadIdx.x; c < NB; c += 64 * W) {
        T sum = colred[0][c];
#pragma unroll
        for (int w = 1; w < W; ++w) sum = E::add(sum, colred[w][c]);
        args.colpart[(long long)slot * NB + c] = sum;
    }
}

// ---------------------------------------------------------------------------
// Ordered merge and epilogue: y_i := beta*y_i + alpha*total_i, where total_i
// adds the row partials of row i in ascending panel order, then the column
// partials of column i in ascending slot order.  SPLIT waves share a block
// of 64 rows: wave g sums the partials k with k % SPLIT == g (the same fixed
// sequence every run), and the SPLIT subtotals are then added by a fixed
// pairwise tree.  beta == 0 never reads y.
template <class T>
struct MergeArgs {
    const T* rowpart;
    const T* colpart;
    const int* slot_base;  // [P+1]: slots of panel p are [slot_base[p], slot_base[p+1])
    T* y;
    long long incy;
    long long ky;          // storage index of logical element 0 of y
    T alpha;
    T beta;
    int n;
    int P;
    int NB;
    int upper;
    int beta_zero;
};

template <class T, int SPLIT>
__global__ __launch_bounds__(64 * SPLIT) void symv_merge(MergeArgs<T> a)
{
    using E = Elem<T>;
    __shared__ T part[SPLIT][64];
    const int lane = threadIdx.x & 63;
    const int g = threadIdx.x >> 6;
    const int i = blockIdx.x * 64 + lane;
    T acc = E::zero();
    if (i < a.n) {
        const int pi = i / a.NB;
        const int p_lo = a.upper ? pi : 0;
        const int p_hi = a.upper ? a.P - 1 : pi;
        const int s_lo = a.slot_base[pi];
        const int s_hi = a.slot_base[pi + 1];
        const int nrow = p_hi - p_lo + 1;
        const int ntot = nrow + (s_hi - s_lo);
        const int ci = i - pi * a.NB;
        const T* __restrict__ rp = a.rowpart + (long long)p_lo * a.n + i;
        const T* __restrict__ cp = a.colpart + (long long)s_lo * a.NB + ci;
        acc = ordered_batch_sum<T, MERGE_BATCH>(acc, g, ntot, SPLIT, [&](int k) {
            return k < nrow ? rp + (long long)k * a.n : cp + (long long)(k - nrow) * a.NB;
        });
    }
    part[g][lane] = acc;
    __syncthreads();
#pragma unroll
    for (int w = SPLIT / 2; w >= 1; w >>= 1) {
        if (g < w) part[g][lane] = E::add(part[g][lane], part[g + w][lane]);
        __syncthreads();
    }
    if (g == 0 && i < a.n) {
        const T tot = part[0][lane];
        T* yp = a.y + a.ky + (long long)i * a.incy;
        T r = E::mul(a.alpha, tot);
        if (!a.beta_zero) r = E::add(r, E::mul(a.beta, *yp));
        *yp = r;
    }
}

// y := beta*y (alpha == 0); beta == 0 writes zeros without reading y.
template <class T>
__global__ __launch_bounds__(256) void symv_scale(T* y, long long incy, long long ky, int n,
                                                  T beta, int beta_zero)
{
    using E = Elem<T>;
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
        T* yp = y + ky + i * incy;
        *yp = beta_zero ? E::zero() : E::mul(beta, *yp);
    }
}

// Contiguous copy of a strided x (incx != 1).
template <class T>
__global__ __launch_bounds__(256) void symv_gather(const T* x, long long incx, long long kx,
                                                   int n, T* out)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = x[kx + i * incx];
}

}  // namespace xsymv
