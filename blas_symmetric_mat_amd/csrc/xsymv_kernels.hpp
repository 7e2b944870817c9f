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

// One workgroup's tile.  rows [r0, r1), panel p, colpart slot, flags.
struct TileDesc {
    int p;
    int r0;
    int r1;
    int slot_flags;  // slot << 2 | flags
};
enum : int { TILE_MASKED = 1 };

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
    const bool masked = (d.slot_flags & TILE_MASKED) != 0;
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
        xc[c] = (cw0 + c < n) ? x[cw0 + c] : E::zero();
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
#pragma unroll
        for (int k = 0; k < V; ++k) {
            racc[s][k] = E::zero();
            const int r = r0 + s * H + lane * V + k;
            xr[s][k] = (r < r1) ? x[r] : E::zero();
        }
    }

    if (!masked) {
        // Full tile: R rows, all NB columns stored, strictly off the diagonal.
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
    } else {
        // Diagonal or ragged tile: element-wise predicates; elements outside
        // the stored triangle or beyond n are never loaded.  The column loop
        // is not unrolled (this path is a small share of the work).
#pragma nounroll
        for (int c = 0; c < CW; ++c) {
            const int col = cw0 + c;
            if (col >= n) break;  // wave-uniform
            const T* __restrict__ Ac = A + (long long)col * lda;
            const T xcol = x[col];
            T csum = E::zero();
#pragma unroll
            for (int s = 0; s < S; ++s) {
                if (r0 + s * H < r1) {  // workgroup-uniform
#pragma unroll
                    for (int k = 0; k < V; ++k) {
                        const int r = r0 + s * H + lane * V + k;
                        const bool st = (r < r1) && (UPPER ? (r <= col) : (r >= col));
                        if (st) {
                            if (r == col) {
                                racc[s][k] = E::mac(racc[s][k], E::diag_load(Ac + r), xcol);
                            } else {
                                const T a = Ac[r];
                                racc[s][k] = E::mac(racc[s][k], a, xcol);
                                csum = E::macc(csum, a, xr[s][k]);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int cc = 0; cc < CW; ++cc) cacc[cc] = E::sel(cc == c, csum, cacc[cc]);
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
// partials of column i in ascending slot order.  Four waves share a row block:
// wave g sums the partials k with k % 4 == g (same fixed sequence every run);
// the four subtotals are then added in wave order.  beta == 0 never reads y.
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

template <class T>
__global__ __launch_bounds__(256) void symv_merge(MergeArgs<T> a)
{
    using E = Elem<T>;
    __shared__ T part[4][64];
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
        for (int k = g; k < ntot; k += 4) {
            T v;
            if (k < nrow)
                v = a.rowpart[(long long)(p_lo + k) * a.n + i];
            else
                v = a.colpart[(long long)(s_lo + k - nrow) * a.NB + ci];
            acc = E::add(acc, v);
        }
    }
    part[g][lane] = acc;
    __syncthreads();
    if (g == 0 && i < a.n) {
        T tot = E::add(E::add(part[0][lane], part[1][lane]), E::add(part[2][lane], part[3][lane]));
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
