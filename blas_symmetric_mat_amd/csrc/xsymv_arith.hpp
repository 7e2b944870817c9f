// xsymv_arith.hpp -- element types and per-element arithmetic for the gfx950
// SYMV/HEMV kernels.
//
// Element types follow the CUDA-xSYMV report, §2.2: real float / double,
// interleaved complex (re, im) pairs for the Hermitian products, and the
// double-double type (hi, lo), a value being the unevaluated sum hi + lo.
//
// Every type provides, for the kernels:
//   VEC             elements per 16-byte lane load
//   SCALAR_X        read x at a column's (wave-uniform) index with scalar
//                   loads in the row-strip kernel for uplo = L; measured per
//                   type: it helps the fp32 types and costs the fp64-based
//                   ones
//   zero()
//   mac(acc, a, x)  acc + a*x          (the row role of a stored element)
//   macc(acc, a, x) acc + conj(a)*x    (the column role: the mirrored element)
//   add(a, b), mul(a, b)
//   diag_load(p)    the diagonal element (Hermitian: the real word only)
//   DIAG_WORDS      leading 32-bit words of an element that a diagonal
//                   element's value uses (Hermitian: the real word only)
//   load16(p, out)  VEC consecutive elements, one 16-byte load, dword aligned
//   shfl_xor(v, m)  exchange with lane ^ m inside a wave64
//   sel(c, a, b)    c ? a : b, word by word (keeps values in registers)
//   load_any(p, diag) the element at p; if `diag`, the diagonal value
//                   (Hermitian: the real word, twice read, never the
//                   imaginary word) -- branch-free, so loads can be batched
//
// Double-double arithmetic is written from the published error-free
// transformations: Knuth's TwoSum, Dekker's FastTwoSum, TwoProd with one
// fused multiply-add, and the accurate double-double addition and the
// multiplication of Hida, Li and Bailey (the report's reference [14]).  The
// accumulating multiply-add (mac, macc) takes that library's cheaper addition
// instead -- one TwoSum of the high words -- which is what the report's count
// of about 21 double operations per double-double operation (§2.2) implies;
// merges and reductions keep the accurate addition.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xsymv {

struct cf32 { float re, im; };
struct cf64 { double re, im; };
struct ddreal { double hi, lo; };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const void* p)
{
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
    if constexpr (NT)
        return __builtin_nontemporal_load(q);
    else
        return *q;
}

// 16 bytes at byte offset `off` of a raw buffer: dwords at or past the
// buffer's byte count read as zero and touch no memory (range checked per
// dword on gfx950), so one 16-byte load can end exactly at a row bound.
constexpr int BUF_DWORD3 = 0x00020000;  // raw buffer, 32-bit data format

// Buffer descriptor of `bytes` bytes at `base`; both must be the same in
// every lane of the wave (they are read from the first active lane, so the
// descriptor lives in scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes)
{
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    void* q = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, __builtin_amdgcn_readfirstlane(bytes),
                                             BUF_DWORD3);
}

template <bool NT>
__device__ __forceinline__ u32x4 bld16(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? 2 : 0));
}

__device__ __forceinline__ float shfl_xor_f(float v, int m)
{
    return __shfl_xor(v, m, 64);
}
__device__ __forceinline__ double shfl_xor_d(double v, int m)
{
    return __shfl_xor(v, m, 64);
}

template <class T> struct Elem;

// ------------------------------------------------------------------ float
template <> struct Elem<float> {
    static constexpr int VEC = 4;
    static constexpr bool SCALAR_X = true;
    static constexpr int DIAG_WORDS = 1;
    __device__ static float zero() { return 0.0f; }
    __device__ static float mac(float acc, float a, float x) { return __builtin_fmaf(a, x, acc); }
    __device__ static float macc(float acc, float a, float x) { return __builtin_fmaf(a, x, acc); }
    __device__ static float add(float a, float b) { return a + b; }
    __device__ static float mul(float a, float b) { return a * b; }
    __device__ static float diag_load(const float* p) { return *p; }
    __device__ static void unpack(u32x4 v, float (&o)[VEC])
    {
        o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
        o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
    }
    template <bool NT>
    __device__ static void load16(const float* p, float (&o)[VEC]) { unpack(ld16<NT>(p), o); }
    template <bool NT>
    __device__ static void bload16(__amdgpu_buffer_rsrc_t r, int off, float (&o)[VEC])
    {
        unpack(bld16<NT>(r, off), o);
    }
    __device__ static float shfl_xor(float v, int m) { return shfl_xor_f(v, m); }
    __device__ static float sel(bool c, float a, float b) { return c ? a : b; }
    __device__ static float load_any(const float* p, bool) { return *p; }
    __device__ static bool is_zero(float a) { return a == 0.0f; }
    __device__ static bool is_one(float a) { return a == 1.0f; }
};

// ----------------------------------------------------------------- double
template <> struct Elem<double> {
    static constexpr int VEC = 2;
    static constexpr bool SCALAR_X = false;
    static constexpr int DIAG_WORDS = 2;
    __device__ static double zero() { return 0.0; }
    __device__ static double mac(double acc, double a, double x) { return __builtin_fma(a, x, acc); }
    __device__ static double macc(double acc, double a, double x) { return __builtin_fma(a, x, acc); }
    __device__ static double add(double a, double b) { return a + b; }
    __device__ static double mul(double a, double b) { return a * b; }
    __device__ static double diag_load(const double* p) { return *p; }
    __device__ static void unpack(u32x4 v, double (&o)[VEC])
    {
        o[0] = __hiloint2double((int)v.y, (int)v.x);
        o[1] = __hiloint2double((int)v.w, (int)v.z);
    }
    template <bool NT>
    __device__ static void load16(const double* p, double (&o)[VEC]) { unpack(ld16<NT>(p), o); }
    template <bool NT>
    __device__ static void bload16(__amdgpu_buffer_rsrc_t r, int off, double (&o)[VEC])
    {
        unpack(bld16<NT>(r, off), o);
    }
    __device__ static double shfl_xor(double v, int m) { return shfl_xor_d(v, m); }
    __device__ static double sel(bool c, double a, double b) { return c ? a : b; }
    __device__ static double load_any(const double* p, bool) { return *p; }
    __device__ static bool is_zero(double a) { return a == 0.0; }
    __device__ static bool is_one(double a) { return a == 1.0; }
};

// -------------------------------------------------------- complex float
template <> struct Elem<cf32> {
    static constexpr int VEC = 2;
    static constexpr bool SCALAR_X = true;
    static constexpr int DIAG_WORDS = 1;
    __device__ static cf32 zero() { return {0.0f, 0.0f}; }
    // acc + a*x
    __device__ static cf32 mac(cf32 acc, cf32 a, cf32 x)
    {
        acc.re = __builtin_fmaf(a.re, x.re, acc.re);
        acc.re = __builtin_fmaf(-a.im, x.im, acc.re);
        acc.im = __builtin_fmaf(a.re, x.im, acc.im);
        acc.im = __builtin_fmaf(a.im, x.re, acc.im);
        return acc;
    }
    // acc + conj(a)*x
    __device__ static cf32 macc(cf32 acc, cf32 a, cf32 x)
    {
        acc.re = __builtin_fmaf(a.re, x.re, acc.re);
        acc.re = __builtin_fmaf(a.im, x.im, acc.re);
        acc.im = __builtin_fmaf(a.re, x.im, acc.im);
        acc.im = __builtin_fmaf(-a.im, x.re, acc.im);
        return acc;
    }
    __device__ static cf32 add(cf32 a, cf32 b) { return {a.re + b.re, a.im + b.im}; }
    __device__ static cf32 mul(cf32 a, cf32 b)
    {
        return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re};
    }
    __device__ static cf32 diag_load(const cf32* p) { return {p->re, 0.0f}; }
    __device__ static void unpack(u32x4 v, cf32 (&o)[VEC])
    {
        o[0] = {__uint_as_float(v.x), __uint_as_float(v.y)};
        o[1] = {__uint_as_float(v.z), __uint_as_float(v.w)};
    }
    template <bool NT>
    __device__ static void load16(const cf32* p, cf32 (&o)[VEC]) { unpack(ld16<NT>(p), o); }
    template <bool NT>
    __device__ static void bload16(__amdgpu_buffer_rsrc_t r, int off, cf32 (&o)[VEC])
    {
        unpack(bld16<NT>(r, off), o);
    }
    __device__ static cf32 shfl_xor(cf32 v, int m)
    {
        return {shfl_xor_f(v.re, m), shfl_xor_f(v.im, m)};
    }
    __device__ static cf32 sel(bool c, cf32 a, cf32 b)
    {
        return {c ? a.re : b.re, c ? a.im : b.im};
    }
    __device__ static cf32 load_any(const cf32* p, bool diag)
    {
        const float re = p->re;
        const float im = *(diag ? &p->re : &p->im);
        return {re, diag ? 0.0f : im};
    }
    __device__ static bool is_zero(cf32 a) { return a.re == 0.0f && a.im == 0.0f; }
    __device__ static bool is_one(cf32 a) { return a.re == 1.0f && a.im == 0.0f; }
};

// ------------------------------------------------------- complex double
template <> struct Elem<cf64> {
    static constexpr int VEC = 1;
    static constexpr bool SCALAR_X = false;
    static constexpr int DIAG_WORDS = 2;
    __device__ static cf64 zero() { return {0.0, 0.0}; }
    __device__ static cf64 mac(cf64 acc, cf64 a, cf64 x)
    {
        acc.re = __builtin_fma(a.re, x.re, acc.re);
        acc.re = __builtin_fma(-a.im, x.im, acc.re);
        acc.im = __builtin_fma(a.re, x.im, acc.im);
        acc.im = __builtin_fma(a.im, x.re, acc.im);
        return acc;
    }
    __device__ static cf64 macc(cf64 acc, cf64 a, cf64 x)
    {
        acc.re = __builtin_fma(a.re, x.re, acc.re);
        acc.re = __builtin_fma(a.im, x.im, acc.re);
        acc.im = __builtin_fma(a.re, x.im, acc.im);
        acc.im = __builtin_fma(-a.im, x.re, acc.im);
        return acc;
    }
    __device__ static cf64 add(cf64 a, cf64 b) { return {a.re + b.re, a.im + b.im}; }
    __device__ static cf64 mul(cf64 a, cf64 b)
    {
        return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re};
    }
    __device__ static cf64 diag_load(const cf64* p) { return {p->re, 0.0}; }
    __device__ static void unpack(u32x4 v, cf64 (&o)[VEC])
    {
        o[0] = {__hiloint2double((int)v.y, (int)v.x), __hiloint2double((int)v.w, (int)v.z)};
    }
    template <bool NT>
    __device__ static void load16(const cf64* p, cf64 (&o)[VEC]) { unpack(ld16<NT>(p), o); }
    template <bool NT>
    __device__ static void bload16(__amdgpu_buffer_rsrc_t r, int off, cf64 (&o)[VEC])
    {
        unpack(bld16<NT>(r, off), o);
    }
    __device__ static cf64 shfl_xor(cf64 v, int m)
    {
        return {shfl_xor_d(v.re, m), shfl_xor_d(v.im, m)};
    }
    __device__ static cf64 sel(bool c, cf64 a, cf64 b)
    {
        return {c ? a.re : b.re, c ? a.im : b.im};
    }
    __device__ static cf64 load_any(const cf64* p, bool diag)
    {
        const double re = p->re;
        const double im = *(diag ? &p->re : &p->im);
        return {re, diag ? 0.0 : im};
    }
    __device__ static bool is_zero(cf64 a) { return a.re == 0.0 && a.im == 0.0; }
    __device__ static bool is_one(cf64 a) { return a.re == 1.0 && a.im == 0.0; }
};

// -------------------------------------------------------- double-double
// TwoSum: s + e == a + b exactly, for any doubles a, b.
__device__ __forceinline__ ddreal dd_two_sum(double a, double b)
{
    double s = a + b;
    double v = s - a;
    double e = (a - (s - v)) + (b - v);
    return {s, e};
}
// FastTwoSum: exact when |a| >= |b| (or a == 0).
__device__ __forceinline__ ddreal dd_fast_two_sum(double a, double b)
{
    double s = a + b;
    return {s, b - (s - a)};
}
// Accurate addition: both word pairs summed exactly, renormalised twice.
__device__ __forceinline__ ddreal dd_add(ddreal a, ddreal b)
{
    ddreal s = dd_two_sum(a.hi, b.hi);
    ddreal t = dd_two_sum(a.lo, b.lo);
    s = dd_fast_two_sum(s.hi, s.lo + t.hi);
    return dd_fast_two_sum(s.hi, s.lo + t.lo);
}
// Multiplication: exact product of the high words (one fma gives its error),
// plus the two cross products, renormalised.
__device__ __forceinline__ ddreal dd_mul(ddreal a, ddreal b)
{
    double p = a.hi * b.hi;
    double e = __builtin_fma(a.hi, b.hi, -p);
    e = __builtin_fma(a.hi, b.lo, e);
    e = __builtin_fma(a.lo, b.hi, e);
    return dd_fast_two_sum(p, e);
}

// Multiply-add for accumulations, acc + a*b in 15 double operations: the
// product's error words (the fma-exact error of hi*hi plus both cross
// products) are not renormalised but added to acc.lo, and one TwoSum joins the
// high words before a final FastTwoSum.  With u = 2^-53, the product errs
// by at most about 6u^2|a||b| (two fma roundings, lo*lo dropped) and the
// addition by u^2(3|acc| + 7|a||b|): not relative to a cancelled sum, as the
// accurate addition's error is, but a chain of k such steps stays within
// about (3k + 13)u^2 * sum|a_j||b_j|, inside the componentwise bound
// 4*n*2^-104*(|alpha||S||x| + |beta||y|) = 16*n*u^2*(...) that the results
// are held to.
__device__ __forceinline__ ddreal dd_madd(ddreal acc, ddreal a, ddreal b)
{
    const double p = a.hi * b.hi;
    double e = __builtin_fma(a.hi, b.hi, -p);
    e = __builtin_fma(a.hi, b.lo, e);
    e = __builtin_fma(a.lo, b.hi, e);
    const ddreal s = dd_two_sum(acc.hi, p);
    return dd_fast_two_sum(s.hi, s.lo + (acc.lo + e));
}

template <> struct Elem<ddreal> {
    static constexpr int VEC = 1;
    static constexpr bool SCALAR_X = false;
    static constexpr int DIAG_WORDS = 4;
    __device__ static ddreal zero() { return {0.0, 0.0}; }
    __device__ static ddreal mac(ddreal acc, ddreal a, ddreal x) { return dd_madd(acc, a, x); }
    __device__ static ddreal macc(ddreal acc, ddreal a, ddreal x) { return dd_madd(acc, a, x); }
    __device__ static ddreal add(ddreal a, ddreal b) { return dd_add(a, b); }
    __device__ static ddreal mul(ddreal a, ddreal b) { return dd_mul(a, b); }
    __device__ static ddreal diag_load(const ddreal* p) { return *p; }
    __device__ static void unpack(u32x4 v, ddreal (&o)[VEC])
    {
        o[0] = {__hiloint2double((int)v.y, (int)v.x), __hiloint2double((int)v.w, (int)v.z)};
    }
    template <bool NT>
    __device__ static void load16(const ddreal* p, ddreal (&o)[VEC]) { unpack(ld16<NT>(p), o); }
    template <bool NT>
    __device__ static void bload16(__amdgpu_buffer_rsrc_t r, int off, ddreal (&o)[VEC])
    {
        unpack(bld16<NT>(r, off), o);
    }
    __device__ static ddreal shfl_xor(ddreal v, int m)
    {
        return {shfl_xor_d(v.hi, m), shfl_xor_d(v.lo, m)};
    }
    __device__ static ddreal sel(bool c, ddreal a, ddreal b)
    {
        return {c ? a.hi : b.hi, c ? a.lo : b.lo};
    }
    __device__ static ddreal load_any(const ddreal* p, bool) { return *p; }
    __device__ static bool is_zero(ddreal a) { return a.hi == 0.0 && a.lo == 0.0; }
    __device__ static bool is_one(ddreal a) { return a.hi == 1.0 && a.lo == 0.0; }
};

// ---------------------------------------------------- buffer stores, conj
// One element at byte offset `off` of a raw buffer (4, 8 or 16 bytes);
// offsets at or past the buffer's byte count load zero / store nothing.
template <class T>
__device__ __forceinline__ T bload1(__amdgpu_buffer_rsrc_t r, int off)
{
    if constexpr (sizeof(T) == 4)
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    else if constexpr (sizeof(T) == 8)
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    else
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <class T, bool NT>
__device__ __forceinline__ void bstore1(__amdgpu_buffer_rsrc_t r, int off, T v)
{
    typedef unsigned int v2u __attribute__((ext_vector_type(2)));
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    if constexpr (sizeof(T) == 4)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), r, off, 0,
                                              NT ? 2 : 0);
    else if constexpr (sizeof(T) == 8)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, v), r, off, 0, NT ? 2 : 0);
    else
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, off, 0, NT ? 2 : 0);
}

// 16 bytes (VEC consecutive elements) stored at byte offset `off`; dwords at
// or past the buffer's byte count are dropped.
template <class T, bool NT>
__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, int off,
                                         const T (&o)[Elem<T>::VEC])
{
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    struct Pack {
        T v[Elem<T>::VEC];
    } pk;
    static_assert(sizeof(Pack) == 16, "16-byte vector");
#pragma unroll
    for (int k = 0; k < Elem<T>::VEC; ++k) pk.v[k] = o[k];
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, pk), r, off, 0, NT ? 2 : 0);
}

__device__ __forceinline__ float elem_conj(float a) { return a; }
__device__ __forceinline__ double elem_conj(double a) { return a; }
__device__ __forceinline__ ddreal elem_conj(ddreal a) { return a; }
__device__ __forceinline__ cf32 elem_conj(cf32 a) { return {a.re, -a.im}; }
__device__ __forceinline__ cf64 elem_conj(cf64 a) { return {a.re, -a.im}; }

}  // namespace xsymv
