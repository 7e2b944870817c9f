// xsyr2_strip.hpp -- symmetric / Hermitian rank-2 update on gfx950:
//   A := alpha*x*y^H + conj(alpha)*y*x^H + A   on the stored triangle
// (real and double-double: A := alpha*x*y^T + alpha*y*x^T + A).
//
// The CUDA-xSYMV report's §5 carries its approach to other Level-2 BLAS; the
// rank-2 update is SYMV's partner in reductions to tridiagonal form and reads
// the same one triangle, here read and written once.  Every stored element
// is updated by exactly one lane with the BLAS reference order -- per column
// j: t1 = alpha*conj(y_j), t2 = conj(alpha*x_j), a := (a + x_i*t1) + y_i*t2;
// the Hermitian diagonal becomes Re(a) + Re(x_j*t1 + y_j*t2) with a zero
// imaginary part -- so no reduction is needed and results do not depend on
// the work split.
//
// Work split: the row-strip plan of the symmetric kernels (strips of R rows,
// the strips' columns concatenated and cut into pieces of equal cost over the
// resident workgroups).  Per column the W waves of a workgroup cover one
// contiguous run of R rows.  Loads and stores are raw-buffer operations on one
// descriptor per column and wave, whose byte count ends at the stored bound
// (L: row n; U: the diagonal, inclusive), so the ragged last strip and the
// whole upper band are 16-byte operations and nothing outside the triangle
// is read or written.  The lower band (rows around the diagonal) needs a
// lower bound as well.  For fp32 there the one lane per column whose vector
// holds both unstored rows and the diagonal reads and writes the 16 bytes
// that start at the diagonal instead (rows of the next lane's vector among
// them get, from both lanes, the same bytes), and vectors with no stored row
// are moved past the byte count (no access); the other types go element by
// element, with the offset of an unstored row moved past the byte count.
#pragma once

#include "xsymv_strip.hpp"

namespace xsymv {

template <class T>
struct Syr2Args {
    T* A;
    const T* x;  // contiguous
    const T* y;  // contiguous
    const StripBlock* blocks;
    const int* strip_base;  // [NS+1]
    long long lda;
    T alpha;
    int n;
};

// The updated element (HERM: the Hermitian diagonal rule when `diag`).
template <class T, bool HERM>
__device__ __forceinline__ T syr2_elem(T a, T xi, T yi, T t1, T t2, bool diag)
{
    using E = Elem<T>;
    const T off = E::add(E::add(a, E::mul(xi, t1)), E::mul(yi, t2));
    if constexpr (HERM) {
        const T s = E::add(E::mul(xi, t1), E::mul(yi, t2));
        T d = a;
        d.re = a.re + s.re;
        d.im = 0;
        return E::sel(diag, d, off);
    } else {
        (void)diag;
        return off;
    }
}

template <class T, bool UPPER, bool HERM, int W, int SW, int G, bool NT>
__global__ __launch_bounds__(64 * W) void syr2_strip(Syr2Args<T> a)
{
    using E = Elem<T>;
    constexpr int V = E::VEC;
    constexpr int H = 64 * V;
    constexpr int RW = SW * H;  // rows per wave
    constexpr int R = W * RW;
    constexpr int ES = (int)sizeof(T);
    constexpr int FAR = 0x7fffff00;  // an offset past every byte count
    // L band in whole vectors: measured, it pays for the four-element vectors
    // of fp32 (SSYR2 L n = 32768 942 -> 856 us) and costs the two-element
    // ones about 1 % (DSYR2 L), so those keep the element-wise band
    constexpr bool VBAND = !UPPER && V >= 4;

    const StripBlock bd = a.blocks[blockIdx.x];
    const int n = a.n;
    const long long lda = a.lda;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    T* __restrict__ A = a.A;
    const T* __restrict__ x = a.x;
    const T* __restrict__ y = a.y;
    const T alpha = a.alpha;

    int u = bd.u0;
    int strip = bd.strip0;
    while (u < bd.u1) {  // workgroup-uniform: one segment per iteration
        const int sb0 = a.strip_base[strip];
        const int useg = min(bd.u1, a.strip_base[strip + 1]);
        const int rs0 = strip * R;
        const int rs1 = min(n, rs0 + R);
        const int coff = (UPPER ? rs0 : 0) - sb0;  // column = sequence position + coff
        const int rw = rs0 + wave * RW;            // this wave's first row
        if (rw < rs1) {                            // wave-uniform
            T xr[SW][V], yr[SW][V];
            // L: x and y at the next lane's rows (the rows a vector moved to
            // the diagonal reaches; past n they are never stored)
            constexpr int NV = VBAND ? V : 1;
            T xn[SW][NV], yn[SW][NV];
#pragma unroll
            for (int s = 0; s < SW; ++s) {
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const int r = rw + s * H + lane * V + k;
                    const int rc = r < rs1 ? r : rs1 - 1;
                    xr[s][k] = x[rc];
                    yr[s][k] = y[rc];
                }
                if constexpr (VBAND) {
#pragma unroll
                    for (int k = 0; k < V; ++k) {
                        const int r = rw + s * H + lane * V + V + k;
                        const int rc = r < n ? r : n - 1;
                        xn[s][k] = x[rc];
                        yn[s][k] = y[rc];
                    }
                }
            }
#pragma unroll 1
            for (int g0 = u; g0 < useg; g0 += G) {
                const int jg = g0 + coff;
                const int ng = min(G, useg - g0);
                // no stored element of the group in this wave's rows
                const bool empty = UPPER ? (rw > jg + ng - 1) : (rw + RW <= jg);
                if (empty) continue;  // wave-uniform; no barriers in this kernel
                const bool band = !UPPER && rw <= jg + ng - 1;
                T t1[G], t2[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int cc = g < ng ? jg + g : jg;
                    const T xj = x[cc], yj = y[cc];
                    t1[g] = E::mul(alpha, HERM ? elem_conj(yj) : yj);
                    t2[g] = HERM ? elem_conj(E::mul(alpha, xj)) : E::mul(alpha, xj);
                }
                if (!band) {
                    // whole 16-byte vectors, bounded above by the stored rows
                    __amdgpu_buffer_rsrc_t rsr[G];
                    T av[G][SW][V];
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const int cc = g < ng ? jg + g : jg;
                        const int bound = UPPER ? cc + 1 : n;
                        const int rows = g < ng ? min(RW, max(0, bound - rw)) : 0;
                        rsr[g] = make_rsrc(A + (long long)cc * lda + rw, rows * ES);
#pragma unroll
                        for (int s = 0; s < SW; ++s)
                            E::template bload16<NT>(rsr[g], (s * H + lane * V) * ES, av[g][s]);
                    }
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int s = 0; s < SW; ++s) {
#pragma unroll
                            for (int k = 0; k < V; ++k) {
                                const int r = rw + s * H + lane * V + k;
                                av[g][s][k] = syr2_elem<T, HERM>(av[g][s][k], xr[s][k], yr[s][k],
                                                                 t1[g], t2[g], r == jg + g);
                            }
                            bstore16<T, NT>(rsr[g], (s * H + lane * V) * ES, av[g][s]);
                        }
                } else if constexpr (VBAND) {
                    // lower band, whole vectors: a vector with no stored row
                    // goes past the byte count; the vector that holds the
                    // diagonal and rows above it is replaced by the V rows
                    // starting at the diagonal (4- or 8-byte aligned), whose
                    // rows past the lane's own are the next lane's, updated
                    // to the same bytes there
                    __amdgpu_buffer_rsrc_t rsr[G];
                    T av[G][SW][V];
                    int off[G][SW];
                    int sh[G][SW];  // rows the vector starts below the lane's first row
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const int col = g < ng ? jg + g : jg;
                        const int rows = g < ng ? min(RW, max(0, n - rw)) : 0;
                        rsr[g] = make_rsrc(A + (long long)col * lda + rw, rows * ES);
#pragma unroll
                        for (int s = 0; s < SW; ++s) {
                            const int rf = rw + s * H + lane * V;  // the lane's first row
                            const bool whole = rf >= col;
                            const bool moved = !whole && rf + V > col;
                            sh[g][s] = moved ? col - rf : 0;
                            off[g][s] = whole ? (rf - rw) * ES : moved ? (col - rw) * ES : FAR;
                            E::template bload16<NT>(rsr[g], off[g][s], av[g][s]);
                        }
                    }
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int s = 0; s < SW; ++s) {
                            const int rf = rw + s * H + lane * V;
#pragma unroll
                            for (int k = 0; k < V; ++k) {
                                // element k is row rf + sh + k
                                T xi = xr[s][k], yi = yr[s][k];
#pragma unroll
                                for (int d = 1; d < V; ++d) {
                                    const int q = k + d;
                                    const T xs = q < V ? xr[s][q % V] : xn[s][q % V];
                                    const T ys = q < V ? yr[s][q % V] : yn[s][q % V];
                                    xi = E::sel(sh[g][s] == d, xs, xi);
                                    yi = E::sel(sh[g][s] == d, ys, yi);
                                }
                                const int col = jg + g;
                                av[g][s][k] = syr2_elem<T, HERM>(av[g][s][k], xi, yi, t1[g], t2[g],
                                                                 rf + sh[g][s] + k == col);
                            }
                            bstore16<T, NT>(rsr[g], off[g][s], av[g][s]);
                        }
                } else {
                    // lower band, one element per vector: unstored rows
                    // (above the diagonal or past n) moved out of range
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const int col = jg + g;
                        const bool real = g < ng;
                        const auto rsr = make_rsrc(A + (long long)(real ? col : jg) * lda + rw,
                                                   real ? RW * ES : 0);
#pragma unroll
                        for (int s = 0; s < SW; ++s)
#pragma unroll
                            for (int k = 0; k < V; ++k) {
                                const int r = rw + s * H + lane * V + k;
                                const bool st = r >= col && r < n;
                                const int off = st ? (s * H + lane * V + k) * ES : FAR;
                                const T v = bload1<T>(rsr, off);
                                bstore1<T, NT>(rsr, off,
                                               syr2_elem<T, HERM>(v, xr[s][k], yr[s][k], t1[g],
                                                                  t2[g], r == col));
                            }
                    }
                }
            }
        }
        u = useg;
        ++strip;
    }
}

}  // namespace xsymv
