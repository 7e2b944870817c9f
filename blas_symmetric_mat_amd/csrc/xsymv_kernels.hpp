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
// Main streaming kernel.  Template parameters:
//   T      element type; UPPER: stored triangle
//   W      waves per workgroup; CW columns per wave (NB = W*CW)
//   S      stripes of H = 64*VEC rows per tile (R = S*H)
//   NT     non-temporal loads for A (streamed once)
// Every load of A is issued without a data-dependent branch, so the compiler
// can keep many 16-byte loads in flight per wave.  Elements outside the
// stored triangle are never loaded: predicated-off lanes load a stored
// element instead (the diagonal of a valid column) and discard it.
template <class T, bool UPPER, int W, int CW, int S, bool NT>
__global__ __launch_bounds__(64 * W) void symv_tiles(SymvArgs<T> args)
{
    using E = Elem<T>;
    constexpr int V = E::VEC;
    constexpr int H = 64 * V;
    constexpr int R = S * H;
    constexpr int NB = W * CW;

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
    T xr[S][V];
    T xc[CW];
#pragma unroll
    for (int c = 0; c < CW; ++c) {
        cacc[c] = E::zero();
        const int col = cw0 + c;
        const T v = x[col < n ? col : n - 1];
        xc[c] = E::sel(col < n, v, E::zero());
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
#pragma unroll
        for (int k = 0; k < V; ++k) {
            racc[s][k] = E::zero();
            const int r = r0 + s * H + lane * V + k;
            const T v = x[r < r1 ? r : r1 - 1];
            xr[s][k] = E::sel(r < r1, v, E::zero());
        }
    }

    if (kind == TILE_FULL) {
        // R rows, all NB columns stored, strictly off the diagonal.
        const T* __restrict__ Ab = A + (long long)cw0 * lda + r0 + lane * V;
#pragma unroll
        for (int c = 0; c < CW; ++c) {
#pragma unroll
            for (int s = 0; s < S; ++s) {
                T a[V];
                E::template load16<NT>(Ab + c * lda + s * H, a);
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    racc[s][k] = E::mac(racc[s][k], a[k], xc[c]);
                    cacc[c] = E::macc(cacc[c], a[k], xr[s][k]);
                }
            }
        }
    } else if (kind == TILE_RAGGED) {
        // Off the diagonal, but fewer rows than R and/or columns past n.
        // Whole stripes use 16-byte loads; the one partial stripe uses
        // element loads at clamped addresses.
#pragma unroll
        for (int c = 0; c < CW; ++c) {
            const int col = cw0 + c;
            if (col < n) {  // wave-uniform
                const T* __restrict__ Ac = A + (long long)col * lda;
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const int rs = r0 + s * H;
                    if (rs + H <= r1) {  // workgroup-uniform: a whole stripe
                        T a[V];
                        E::template load16<NT>(Ac + rs + lane * V, a);
#pragma unroll
                        for (int k = 0; k < V; ++k) {
                            racc[s][k] = E::mac(racc[s][k], a[k], xc[c]);
                            cacc[c] = E::macc(cacc[c], a[k], xr[s][k]);
                        }
                    } else if (rs < r1) {  // workgroup-uniform: the partial stripe
#pragma unroll
                        for (int k = 0; k < V; ++k) {
                            const int r = rs + lane * V + k;
                            const T v = Ac[r < r1 ? r : r1 - 1];
                            const T a = E::sel(r < r1, v, E::zero());
                            racc[s][k] = E::mac(racc[s][k], a, xc[c]);
                            cacc[c] = E::macc(cacc[c], a, xr[s][k]);
                        }
                    }
                }
            }
        }
    } else {
        // The panel's diagonal block: rows and columns [c0, min(n, c0+NB)).
        // Element (r, col) is stored when r >= col (L) or r <= col (U); the
        // diagonal element counts once (row role only; Hermitian: real part).
#pragma unroll
        for (int c = 0; c < CW; ++c) {
            const int col = cw0 + c;
            const bool colok = col < n;               // wave-uniform
            const int cc = colok ? col : c0;          // a valid column
            const T* __restrict__ Ac = A + (long long)cc * lda;
#pragma unroll
            for (int s = 0; s < S; ++s) {
                if (r0 + s * H < r1) {  // workgroup-uniform
#pragma unroll
                    for (int k = 0; k < V; ++k) {
                        const int r = r0 + s * H + lane * V + k;
                        const bool st = colok && r < r1 && (UPPER ? (r <= col) : (r >= col));
                        const bool dg = (r == col);
                        const T v = E::load_any(Ac + (st ? r : cc), dg || !st);
                        const T a = E::sel(st, v, E::zero());
                        racc[s][k] = E::mac(racc[s][k], a, xc[c]);
                        cacc[c] = E::macc(cacc[c], E::sel(dg, E::zero(), a), xr[s][k]);
                    }
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
#pragma unroll 4
        for (int k = g; k < ntot; k += SPLIT) {
            const T v = (k < nrow) ? rp[(long long)k * a.n] : cp[(long long)(k - nrow) * a.NB];
            acc = E::add(acc, v);
        }
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
