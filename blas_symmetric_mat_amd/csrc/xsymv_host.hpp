// xsymv_host.hpp -- host-side machinery shared by the per-precision
// translation units of libxsymv: tile configurations, tile plans, per-stream
// workspaces, kernel timing and the call driver symv_impl<T>.
//
// Call flow of one product y := alpha*S*x + beta*y (the CUDA-xSYMV report,
// §1 eq.(1), with the BLAS argument list of §2.2 Fig. 5): check the
// arguments before touching the device; quick returns; pick the tile
// configuration for (precision, uplo, n); fetch or build the tile plan;
// enqueue symv_tiles (every stored element read once, used twice) and then
// symv_merge (fixed-order sum of the partials, alpha/beta epilogue) on the
// caller's stream.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <map>
#include <memory>
#include <mutex>
#include <type_traits>
#include <tuple>
#include <vector>

#include "../../include/xsymv.h"
#include "xsymv_kernels.hpp"
#include "xsymv_strip.hpp"
#include "xgemv_strip.hpp"
#include "xsyr2_strip.hpp"
#include "xtrmv_strip.hpp"

namespace xsymv {

constexpr int ERR_HIP = 1000;
constexpr int ERR_WORKSPACE = 2000;  // a caller-installed workspace is too small
constexpr int ERR_STATIC_SIZE = 3000;    // the static array is too small for the call
constexpr int ERR_STATIC_CONFIG = 3001;  // the selected configuration is not a row strip
constexpr int ERR_STATIC_DEVICE = 3002;  // device index beyond the static table

// Device workspace of one (device, stream): library-owned (grown with
// hipMalloc on demand) or installed by the caller (never freed here).
struct Workspace {
    void* ptr = nullptr;
    size_t bytes = 0;
    bool owned = true;
};
constexpr int MERGE_SPLIT = 16;  // waves sharing one 64-row block of the merge
constexpr int STRIP_CBUF = 256;  // columns a strip workgroup buffers before adding waves

#define XSYMV_HIP(expr)                                 \
    do {                                                \
        hipError_t e_ = (expr);                         \
        if (e_ != hipSuccess) return ERR_HIP + (int)e_; \
    } while (0)

// ------------------------------------------------------------ configurations
struct ConfigInfo {
    int W, CW, S, H, NT, XLDS;
    int RUNS;  // 0: symv_tiles; 1: symv_runs; 2: symv_runs with the next run
               // prefetched; 3: symv_block; 4: symv_strip (CW = column group,
               // S = W * stripes per wave, work split by strip height);
               // 5: symv_strip, work split by stored rows + strip height
    int NB() const { return W * CW; }
    bool strip() const { return RUNS >= 4; }
    int R() const { return S * H; }
};

template <class T>
struct KernelSet {
    void (*lower)(SymvArgs<T>);
    void (*upper)(SymvArgs<T>);
    ConfigInfo info;
    void (*strip_lower)(StripArgs<T>) = nullptr;  // strip family only
    void (*strip_upper)(StripArgs<T>) = nullptr;
};

template <class T, int W, int CW, int S, bool NT, bool XLDS>
KernelSet<T> make_set()
{
    return KernelSet<T>{&symv_tiles<T, false, W, CW, S, NT, XLDS>,
                        &symv_tiles<T, true, W, CW, S, NT, XLDS>,
                        ConfigInfo{W, CW, S, 64 * Elem<T>::VEC, NT ? 1 : 0, XLDS ? 1 : 0, 0}};
}

// Block-run configurations: W waves, NB columns, SW stripes per wave, column
// groups of G.  Reported as cols_per_wave = NB / W and stripes = W * SW so
// that NB and R come out as for the other families.
template <class T, int W, int NB, int SW, int G, bool NT>
KernelSet<T> make_block()
{
    return KernelSet<T>{&symv_block<T, false, W, NB, SW, G, NT>,
                        &symv_block<T, true, W, NB, SW, G, NT>,
                        ConfigInfo{W, NB / W, W * SW, 64 * Elem<T>::VEC, NT ? 1 : 0, 0, 3}};
}

// Row-strip, evenly split configurations: W waves, SW stripes per wave,
// column groups of G.
template <class T, int W, int SW, int G, bool NT, int SPLIT = 0>
KernelSet<T> make_strip()
{
    KernelSet<T> k{nullptr, nullptr,
                   ConfigInfo{W, G, W * SW, 64 * Elem<T>::VEC, NT ? 1 : 0, 0, 4 + SPLIT}};
    k.strip_lower = &symv_strip<T, false, W, SW, G, NT, STRIP_CBUF>;
    k.strip_upper = &symv_strip<T, true, W, SW, G, NT, STRIP_CBUF>;
    return k;
}

template <class T, int W, int CW, int S, bool NT, bool PF>
KernelSet<T> make_runs()
{
    return KernelSet<T>{&symv_runs<T, false, W, CW, S, NT, PF>,
                        &symv_runs<T, true, W, CW, S, NT, PF>,
                        ConfigInfo{W, CW, S, 64 * Elem<T>::VEC, NT ? 1 : 0, 1, PF ? 2 : 1}};
}

// Defined in the per-precision translation units.
template <class T> const std::vector<KernelSet<T>>& kernel_sets();
template <> const std::vector<KernelSet<float>>& kernel_sets<float>();
template <> const std::vector<KernelSet<double>>& kernel_sets<double>();
template <> const std::vector<KernelSet<cf32>>& kernel_sets<cf32>();
template <> const std::vector<KernelSet<cf64>>& kernel_sets<cf64>();
template <> const std::vector<KernelSet<ddreal>>& kernel_sets<ddreal>();

template <class T> constexpr int prec_code();
template <> constexpr int prec_code<float>() { return XSYMV_S; }
template <> constexpr int prec_code<double>() { return XSYMV_D; }
template <> constexpr int prec_code<cf32>() { return XSYMV_C; }
template <> constexpr int prec_code<cf64>() { return XSYMV_Z; }
template <> constexpr int prec_code<ddreal>() { return XSYMV_W; }

// Stride class of a leading dimension: 0 when a column is a whole number of
// 64-byte lines (every column starts where the previous one's lines end),
// 1 otherwise (a wave's piece of a column then straddles one line more).
inline int stride_class(long long lda, size_t elem) { return (lda * (long long)elem) % 64 ? 1 : 0; }

// Configuration index for (prec, upper, n, stride class): the last matching
// caller rule, else the built-in rules of that class (falling back to class
// 0), else entry 0.
int pick_config(int prec, bool upper, int n, int cls = 0);

// --------------------------------------------------------------- tile plans
struct Plan {
    int P = 0, NB = 0, ntiles = 0, nslots = 0;
    TileDesc* d_tiles = nullptr;
    int* d_slot_base = nullptr;
    TileDesc* h_tiles = nullptr;  // pinned source of the one upload
    int* h_slot_base = nullptr;
};

// Tiles of the panel decomposition (see xsymv_kernels.hpp).  For every panel:
// the diagonal tile, then the off-diagonal tiles in row order; that is the
// slot order the merge uses.  Dispatch order: diagonal and ragged tiles
// first, then the full tiles.
void build_plan_host(bool upper, int n, int NB, int R, std::vector<TileDesc>& tiles,
                     std::vector<int>& slot_base, int& P);

// Row-strip plan: R-row strips, the column sequence split evenly over G
// workgroups (see xsymv_strip.hpp).
struct StripPlan {
    int NS = 0, G = 0, nseg = 0, R = 0;
    StripBlock* d_blocks = nullptr;
    int* d_strip_base = nullptr;
    int* d_seg_base = nullptr;
    std::vector<int> h_seg_base;  // host copy (the merge takes it as arguments)
    void* h_pinned = nullptr;  // pinned source of the one upload
    // one shard's product: its local columns (see StripArgs)
    int ncol = 0;
    int* d_lcol = nullptr;
    int* d_gloc = nullptr;
    int* d_col0 = nullptr;
};
// lcol (optional): the ascending global columns of a shard's local matrix;
// the strips' sequences then run over local columns (col0: the first local
// column of each strip's sequence).
void build_strip_plan_host(bool upper, int n, int R, int G, int split, std::vector<StripBlock>& blocks,
                           std::vector<int>& strip_base, std::vector<int>& seg_base, int& NS,
                           const std::vector<int>* lcol = nullptr,
                           std::vector<int>* col0 = nullptr);

// Columns of one shard when panels of `panel` columns are dealt to `nshards`
// shards round by round, forward in even rounds and backward in odd ones.
int shard_owner(int panel_index, int nshards);
void shard_columns_host(int n, int panel, int nshards, int shard, std::vector<int>& cols);
int shard_column_count(int n, int panel, int nshards, int shard);

// xGEMV: (strip, column) sequence of NS strips x n columns, equal pieces
// (per-column cost: the strip's rows plus a fixed share).
void build_gemv_plan_host(int m, int n, int R, int G, std::vector<StripBlock>& blocks,
                          std::vector<int>& seg_base, int& NS);

struct DeviceState;
DeviceState* device_state(int dev);
int get_gemv_plan(DeviceState* ds, int m, int n, int R, int G, hipStream_t stream,
                  const StripPlan** out);
int get_strip_plan(DeviceState* ds, int dev, bool upper, int n, int R, int G, int split, hipStream_t stream,
                   const StripPlan** out);
int get_shard_plan(DeviceState* ds, bool upper, int n, int R, int G, int split, int panel,
                   int nshards, int shard, hipStream_t stream, const StripPlan** out);
// Workgroups of `kernel` (block size `threads`) the current device holds at once.
int resident_blocks(const void* kernel, int threads, int* out);
// Both return 0 or ERR_HIP + hipError_t; the caller holds the state's lock.
int get_plan(DeviceState* ds, int dev, bool upper, int n, int NB, int R, hipStream_t stream,
             const Plan** out);
int get_workspace(DeviceState* ds, hipStream_t stream, size_t bytes, void** out);
std::mutex& device_mutex(DeviceState* ds);

inline size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

// Strip workspace layout: [rowpart nseg*R][colpart NS*n][x gathered, n]
template <class T>
size_t strip_workspace_bytes(int nseg, int R, int NS, int n)
{
    return align_up((size_t)nseg * R * sizeof(T)) + align_up((size_t)NS * n * sizeof(T)) +
           align_up((size_t)n * sizeof(T));
}

// Workspace layout: [rowpart P*n][colpart nslots*NB][x gathered, n]
template <class T>
size_t workspace_bytes_for(int P, int n, int nslots, int NB)
{
    return align_up((size_t)P * n * sizeof(T)) + align_up((size_t)nslots * NB * sizeof(T)) +
           align_up((size_t)n * sizeof(T));
}

// ------------------------------------------------------------------- timing
// One timed call: e0 takes the main kernel's own start, e1 its end, e2 the
// end of the merge.  Null events are not taken: all while timing is off; e2
// for a call of one kernel; e1 in whole-call mode (timing mode 2), where no
// event is bound between the two kernels.
struct TimedCall {
    hipEvent_t e0 = nullptr, e1 = nullptr, e2 = nullptr;
};
int timing_enabled();  // the timing mode: 0 off, 1 main kernel and merge, 2 whole call
void timing_push(const TimedCall& c);

// Creates the events of a timed call in timing mode `mode`; `merge`: the call
// has a second kernel.
inline hipError_t timed_call_create(TimedCall& tc, int mode, bool merge = true)
{
    hipError_t e = hipEventCreate(&tc.e0);
    if (e == hipSuccess && (mode == 1 || !merge)) e = hipEventCreate(&tc.e1);
    if (e == hipSuccess && merge) e = hipEventCreate(&tc.e2);
    return e;
}

// Launches kernel `k` (one argument struct) on `stream`.  Given events, they
// take the kernel's own start and end times from its dispatch (HIP's extended
// launch), so that timing puts no marker packet between the kernels of a
// call: a marker between the streaming kernel and its merge delays the merge
// by several microseconds.
template <class A>
hipError_t launch_k(void (*k)(A), dim3 grid, dim3 block, hipStream_t stream, A args,
                    hipEvent_t start = nullptr, hipEvent_t stop = nullptr)
{
    if (start == nullptr && stop == nullptr) {
        k<<<grid, block, 0, stream>>>(args);
        return hipGetLastError();
    }
    void* p[] = {&args};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(k), grid, block, p, 0, stream, start,
                              stop, 0);
}

// ---------------------------------------------------------------- checking
int check_args(char uplo, int n, const void* A, int lda, const void* x, int incx,
               const void* y, int incy, bool* upper);

inline bool host_is_zero(float a) { return a == 0.0f; }
inline bool host_is_zero(double a) { return a == 0.0; }
inline bool host_is_zero(cf32 a) { return a.re == 0.0f && a.im == 0.0f; }
inline bool host_is_zero(cf64 a) { return a.re == 0.0 && a.im == 0.0; }
inline bool host_is_zero(ddreal a) { return a.hi == 0.0 && a.lo == 0.0; }
inline bool host_is_one(float a) { return a == 1.0f; }
inline bool host_is_one(double a) { return a == 1.0; }
inline bool host_is_one(cf32 a) { return a.re == 1.0f && a.im == 0.0f; }
inline bool host_is_one(cf64 a) { return a.re == 1.0 && a.im == 0.0; }
inline bool host_is_one(ddreal a) { return a.hi == 1.0 && a.lo == 0.0; }

inline unsigned blocks_for(long long n, int per) { return (unsigned)((n + per - 1) / per); }

template <class T> T tune_one();
template <> inline float tune_one<float>() { return 1.0f; }
template <> inline double tune_one<double>() { return 1.0; }
template <> inline cf32 tune_one<cf32>() { return {1.0f, 0.0f}; }
template <> inline cf64 tune_one<cf64>() { return {1.0, 0.0}; }
template <> inline ddreal tune_one<ddreal>() { return {1.0, 0.0}; }
template <class T> T tune_zero();
template <> inline float tune_zero<float>() { return 0.0f; }
template <> inline double tune_zero<double>() { return 0.0; }
template <> inline cf32 tune_zero<cf32>() { return {0.0f, 0.0f}; }
template <> inline cf64 tune_zero<cf64>() { return {0.0, 0.0}; }
template <> inline ddreal tune_zero<ddreal>() { return {0.0, 0.0}; }

// Autotuner per element type (specialised in the precision units, where the
// kernels live).
template <class T>
int autotune_for(char uplo, int n, int lda, int reps, hipStream_t stream, int* best_idx,
                 float* ms, int max_cfg);
template <> int autotune_for<float>(char, int, int, int, hipStream_t, int*, float*, int);
template <> int autotune_for<double>(char, int, int, int, hipStream_t, int*, float*, int);
template <> int autotune_for<cf32>(char, int, int, int, hipStream_t, int*, float*, int);
template <> int autotune_for<cf64>(char, int, int, int, hipStream_t, int*, float*, int);
template <> int autotune_for<ddreal>(char, int, int, int, hipStream_t, int*, float*, int);

// --------------------------------------------------------------- the driver
// The strip family's half of a call (the caller holds the device lock).
template <class T>
int strip_run(const KernelSet<T>& ks, bool upper, int n, T alpha, const T* A, int lda,
              const T* x, int incx, long long kx, T beta, int beta_zero, T* y, int incy,
              long long ky, hipStream_t stream, DeviceState* ds, int dev)
{
    const int R = ks.info.R();
    const int threads = 64 * ks.info.W;
    auto kern = upper ? ks.strip_upper : ks.strip_lower;
    int G = 0;
    int rc = resident_blocks((const void*)kern, threads, &G);
    if (rc) return rc;
    const StripPlan* plan = nullptr;
    rc = get_strip_plan(ds, dev, upper, n, R, G, ks.info.RUNS - 4, stream, &plan);
    if (rc) return rc;
    void* ws = nullptr;
    rc = get_workspace(ds, stream, strip_workspace_bytes<T>(plan->nseg, R, plan->NS, n), &ws);
    if (rc) return rc;
    char* base = static_cast<char*>(ws);
    const size_t off_col = align_up((size_t)plan->nseg * R * sizeof(T));
    const size_t off_x = off_col + align_up((size_t)plan->NS * n * sizeof(T));
    T* rowpart = reinterpret_cast<T*>(base);
    T* colpart = reinterpret_cast<T*>(base + off_col);
    T* xg = reinterpret_cast<T*>(base + off_x);
    const T* xin = x;
    if (incx != 1) {
        symv_gather<T><<<blocks_for(n, 256), 256, 0, stream>>>(x, incx, kx, n, xg);
        XSYMV_HIP(hipGetLastError());
        xin = xg;
    }
    TimedCall tc{};
    const int timing = timing_enabled();
    if (timing) {
        XSYMV_HIP(timed_call_create(tc, timing));
    }
    StripArgs<T> sa{A, xin, rowpart, colpart, plan->d_blocks, plan->d_strip_base,
                    (long long)lda, n};
    XSYMV_HIP(launch_k(kern, plan->G, threads, stream, sa, tc.e0, tc.e1));
    StripMergeArgs<T> ma{rowpart, colpart, plan->d_seg_base, y, (long long)incy, ky, alpha, beta,
                         n, plan->NS, R, upper ? 1 : 0, beta_zero};
    XSYMV_HIP((launch_strip_merge<T, MERGE_SPLIT>(ma, n, stream, tc.e2, plan->h_seg_base.data())));
    if (timing) timing_push(tc);
    return 0;
}

// forced_idx >= 0 runs that configuration instead of the selected one.
template <class T>
int symv_run(char uplo, int n, T alpha, const T* A, int lda, const T* x, int incx, T beta,
             T* y, int incy, hipStream_t stream, int forced_idx)
{
    bool upper = false;
    int rc = check_args(uplo, n, A, lda, x, incx, y, incy, &upper);
    if (rc) return rc;
    if (n == 0 || (host_is_zero(alpha) && host_is_one(beta))) return 0;
    const long long ky = incy > 0 ? 0 : (long long)(1 - n) * incy;
    const long long kx = incx > 0 ? 0 : (long long)(1 - n) * incx;
    const int beta_zero = host_is_zero(beta) ? 1 : 0;
    if (host_is_zero(alpha)) {
        symv_scale<T><<<blocks_for(n, 256), 256, 0, stream>>>(y, incy, ky, n, beta, beta_zero);
        XSYMV_HIP(hipGetLastError());
        return 0;
    }

    const int idx = forced_idx >= 0 ? forced_idx
                                    : pick_config(prec_code<T>(), upper, n,
                                                  stride_class(lda, sizeof(T)));
    const KernelSet<T>& ks = kernel_sets<T>()[idx];
    const int NB = ks.info.NB();
    const int R = ks.info.R();

    int dev = 0;
    XSYMV_HIP(hipGetDevice(&dev));
    DeviceState* ds = device_state(dev);
    std::lock_guard<std::mutex> lk(device_mutex(ds));
    if (ks.info.strip())
        return strip_run<T>(ks, upper, n, alpha, A, lda, x, incx, kx, beta, beta_zero, y, incy,
                            ky, stream, ds, dev);
    const Plan* plan = nullptr;
    rc = get_plan(ds, dev, upper, n, NB, R, stream, &plan);
    if (rc) return rc;
    void* ws = nullptr;
    rc = get_workspace(ds, stream, workspace_bytes_for<T>(plan->P, n, plan->nslots, NB), &ws);
    if (rc) return rc;
    char* base = static_cast<char*>(ws);
    const size_t off_col = align_up((size_t)plan->P * n * sizeof(T));
    const size_t off_x = off_col + align_up((size_t)plan->nslots * NB * sizeof(T));
    T* rowpart = reinterpret_cast<T*>(base);
    T* colpart = reinterpret_cast<T*>(base + off_col);
    T* xg = reinterpret_cast<T*>(base + off_x);

    const T* xin = x;
    if (incx != 1) {
        symv_gather<T><<<blocks_for(n, 256), 256, 0, stream>>>(x, incx, kx, n, xg);
        XSYMV_HIP(hipGetLastError());
        xin = xg;
    }

    TimedCall tc{};
    const int timing = timing_enabled();
    if (timing) {
        XSYMV_HIP(timed_call_create(tc, timing));
    }

    SymvArgs<T> sa{A, xin, rowpart, colpart, plan->d_tiles, (long long)lda, n};
    const int threads = 64 * ks.info.W;
    XSYMV_HIP(launch_k(upper ? ks.upper : ks.lower, plan->ntiles, threads, stream, sa, tc.e0,
                       tc.e1));

    MergeArgs<T> ma{rowpart, colpart, plan->d_slot_base, y, (long long)incy, ky, alpha, beta,
                    n, plan->P, NB, upper ? 1 : 0, beta_zero};
    XSYMV_HIP(launch_k(&symv_merge<T, MERGE_SPLIT>, blocks_for(n, 64), 64 * MERGE_SPLIT, stream,
                       ma, nullptr, tc.e2));
    if (timing) timing_push(tc);
    return 0;
}

template <class T>
int symv_impl(char uplo, int n, T alpha, const T* A, int lda, const T* x, int incx, T beta,
              T* y, int incy, hipStream_t stream)
{
    return symv_run<T>(uplo, n, alpha, A, lda, x, incx, beta, y, incy, stream, -1);
}

// ------------------------------------------------------------------ xGEMV
template <class T>
struct GemvKernelSet {
    int W, SW, G, NT;
    void (*k[3])(GemvArgs<T>);  // 'N', 'T', 'C'
    int R() const { return W * SW * 64 * Elem<T>::VEC; }
};

template <class T, int W, int SW, int G, bool NT>
GemvKernelSet<T> make_gemv()
{
    constexpr bool cplx = std::is_same<T, cf32>::value || std::is_same<T, cf64>::value;
    GemvKernelSet<T> k{W, SW, G, NT ? 1 : 0, {}};
    k.k[0] = &gemv_strip<T, 0, W, SW, G, NT, STRIP_CBUF>;
    k.k[1] = &gemv_strip<T, 1, W, SW, G, NT, STRIP_CBUF>;
    k.k[2] = cplx ? &gemv_strip<T, 2, W, SW, G, NT, STRIP_CBUF> : k.k[1];
    return k;
}

template <class T> const std::vector<GemvKernelSet<T>>& gemv_kernel_sets();
int gemv_selected(int prec);  // -1: the built-in choice

// Built-in xGEMV choice per element type: [0 'N', 1 'T' or 'C'][size
// class], the size class from the matrix's element count m*n: below
// 12288^2, below 20000^2, then larger (the orders 8192, 16384 and 32768 --
// 23170 for the 16-byte types -- fall one in each).
struct GemvDefaults {
    int idx[2][3];
};
template <class T> GemvDefaults gemv_defaults();

inline int gemv_size_class(int m, int n)
{
    const long long e = (long long)m * n;
    return e < 12288LL * 12288 ? 0 : e < 20000LL * 20000 ? 1 : 2;
}

template <class T>
int gemv_pick(int tr, int m, int n)
{
    const int sel = gemv_selected(prec_code<T>());
    return sel >= 0 ? sel : gemv_defaults<T>().idx[tr != 0 ? 1 : 0][gemv_size_class(m, n)];
}

int check_gemv_args(char trans, int m, int n, const void* A, int lda, const void* x, int incx,
                    const void* y, int incy, int* tr);

// Workspace of a GEMV call: [partials][x gathered]
template <class T>
size_t gemv_workspace_bytes(int tr, int nseg, int R, int NS, int n, int lenx)
{
    const size_t part = tr == 0 ? (size_t)nseg * R : (size_t)NS * n;
    return align_up(part * sizeof(T)) + align_up((size_t)lenx * sizeof(T));
}

template <class T>
int gemv_run(char trans, int m, int n, T alpha, const T* A, int lda, const T* x, int incx,
             T beta, T* y, int incy, hipStream_t stream, int forced_idx)
{
    int tr = 0;
    int rc = check_gemv_args(trans, m, n, A, lda, x, incx, y, incy, &tr);
    if (rc) return rc;
    if (m == 0 || n == 0 || (host_is_zero(alpha) && host_is_one(beta))) return 0;
    const int leny = tr == 0 ? m : n, lenx = tr == 0 ? n : m;
    const long long ky = incy > 0 ? 0 : (long long)(1 - leny) * incy;
    const long long kx = incx > 0 ? 0 : (long long)(1 - lenx) * incx;
    const int beta_zero = host_is_zero(beta) ? 1 : 0;
    if (host_is_zero(alpha)) {
        symv_scale<T><<<blocks_for(leny, 256), 256, 0, stream>>>(y, incy, ky, leny, beta,
                                                                 beta_zero);
        XSYMV_HIP(hipGetLastError());
        return 0;
    }
    const auto& sets = gemv_kernel_sets<T>();
    const int idx = forced_idx >= 0 ? forced_idx : gemv_pick<T>(tr, m, n);
    const GemvKernelSet<T>& ks = sets[idx];
    const int R = ks.R();
    const int threads = 64 * ks.W;
    auto kern = ks.k[tr];

    int dev = 0;
    XSYMV_HIP(hipGetDevice(&dev));
    DeviceState* ds = device_state(dev);
    std::lock_guard<std::mutex> lk(device_mutex(ds));
    int G = 0;
    rc = resident_blocks((const void*)kern, threads, &G);
    if (rc) return rc;
    const StripPlan* plan = nullptr;
    rc = get_gemv_plan(ds, m, n, R, G, stream, &plan);
    if (rc) return rc;
    void* ws = nullptr;
    rc = get_workspace(ds, stream, gemv_workspace_bytes<T>(tr, plan->nseg, R, plan->NS, n, lenx),
                       &ws);
    if (rc) return rc;
    char* base = static_cast<char*>(ws);
    const size_t part_bytes = align_up((tr == 0 ? (size_t)plan->nseg * R : (size_t)plan->NS * n) *
                                       sizeof(T));
    T* part = reinterpret_cast<T*>(base);
    T* xg = reinterpret_cast<T*>(base + part_bytes);
    const T* xin = x;
    if (incx != 1) {
        symv_gather<T><<<blocks_for(lenx, 256), 256, 0, stream>>>(x, incx, kx, lenx, xg);
        XSYMV_HIP(hipGetLastError());
        xin = xg;
    }
    TimedCall tc{};
    const int timing = timing_enabled();
    if (timing) {
        XSYMV_HIP(timed_call_create(tc, timing));
    }
    GemvArgs<T> ga{A, xin, part, part, plan->d_blocks, (long long)lda, m, n};
    XSYMV_HIP(launch_k(kern, plan->G, threads, stream, ga, tc.e0, tc.e1));
    GemvMergeArgs<T> ma{part, plan->d_seg_base, y, (long long)incy, ky, alpha, beta, leny,
                        plan->NS, R, n, tr, beta_zero};
    XSYMV_HIP(launch_k(&gemv_merge<T, MERGE_SPLIT>, blocks_for(leny, 64), 64 * MERGE_SPLIT,
                       stream, ma, nullptr, tc.e2));
    if (timing) timing_push(tc);
    return 0;
}

template <class T>
size_t gemv_ws_bytes(char trans, int m, int n)
{
    const int tr = (trans == 'N' || trans == 'n') ? 0 : 1;
    if (m <= 0 || n <= 0) return 0;
    const auto& ks = gemv_kernel_sets<T>()[gemv_pick<T>(tr, m, n)];
    int G = 0;
    if (resident_blocks((const void*)ks.k[tr], 64 * ks.W, &G)) return (size_t)-1;
    std::vector<StripBlock> blocks;
    std::vector<int> segb;
    int NS = 0;
    build_gemv_plan_host(m, n, ks.R(), G, blocks, segb, NS);
    return gemv_workspace_bytes<T>(tr, segb[NS], ks.R(), NS, n, tr == 0 ? n : m);
}

// ------------------------------------------------------------ xSYR2 / xHER2
template <class T>
struct Syr2KernelSet {
    int W, SW, G, NT, split;
    void (*k[2])(Syr2Args<T>);  // lower, upper
    int R() const { return W * SW * 64 * Elem<T>::VEC; }
};

template <class T, int W, int SW, int G, bool NT, int SPLIT>
Syr2KernelSet<T> make_syr2()
{
    constexpr bool herm = std::is_same<T, cf32>::value || std::is_same<T, cf64>::value;
    return Syr2KernelSet<T>{W, SW, G, NT ? 1 : 0, SPLIT,
                            {&syr2_strip<T, false, herm, W, SW, G, NT>,
                             &syr2_strip<T, true, herm, W, SW, G, NT>}};
}

template <class T> const std::vector<Syr2KernelSet<T>>& syr2_kernel_sets();
int syr2_selected(int prec);  // -1: the built-in choice

// Built-in xSYR2 / xHER2 choice per element type: [upper][size class of n,
// as for xTRMV: below 12288, below 20000, then larger].
struct Syr2Defaults {
    int idx[2][3];
};
template <class T> Syr2Defaults syr2_defaults();

template <class T>
int syr2_pick(bool upper, int n)
{
    const int sel = syr2_selected(prec_code<T>());
    return sel >= 0 ? sel
                    : syr2_defaults<T>().idx[upper ? 1 : 0][n < 12288 ? 0 : n < 20000 ? 1 : 2];
}
int check_syr2_args(char uplo, int n, const void* x, int incx, const void* y, int incy,
                    const void* A, int lda, bool* upper);

template <class T>
int syr2_run(char uplo, int n, T alpha, const T* x, int incx, const T* y, int incy, T* A,
             int lda, hipStream_t stream, int forced_idx)
{
    bool upper = false;
    int rc = check_syr2_args(uplo, n, x, incx, y, incy, A, lda, &upper);
    if (rc) return rc;
    if (n == 0 || host_is_zero(alpha)) return 0;
    const auto& ks = syr2_kernel_sets<T>()[forced_idx >= 0 ? forced_idx
                                                              : syr2_pick<T>(upper, n)];
    const int R = ks.R();
    const int threads = 64 * ks.W;
    auto kern = ks.k[upper ? 1 : 0];
    int dev = 0;
    XSYMV_HIP(hipGetDevice(&dev));
    DeviceState* ds = device_state(dev);
    std::lock_guard<std::mutex> lk(device_mutex(ds));
    int G = 0;
    rc = resident_blocks((const void*)kern, threads, &G);
    if (rc) return rc;
    const StripPlan* plan = nullptr;
    rc = get_strip_plan(ds, dev, upper, n, R, G, ks.split, stream, &plan);
    if (rc) return rc;
    const T* xin = x;
    const T* yin = y;
    if (incx != 1 || incy != 1) {
        void* ws = nullptr;
        rc = get_workspace(ds, stream, 2 * align_up((size_t)n * sizeof(T)), &ws);
        if (rc) return rc;
        T* xg = static_cast<T*>(ws);
        T* yg = reinterpret_cast<T*>(static_cast<char*>(ws) + align_up((size_t)n * sizeof(T)));
        if (incx != 1) {
            const long long kx = incx > 0 ? 0 : (long long)(1 - n) * incx;
            symv_gather<T><<<blocks_for(n, 256), 256, 0, stream>>>(x, incx, kx, n, xg);
            XSYMV_HIP(hipGetLastError());
            xin = xg;
        }
        if (incy != 1) {
            const long long ky = incy > 0 ? 0 : (long long)(1 - n) * incy;
            symv_gather<T><<<blocks_for(n, 256), 256, 0, stream>>>(y, incy, ky, n, yg);
            XSYMV_HIP(hipGetLastError());
            yin = yg;
        }
    }
    TimedCall tc{};
    const int timing = timing_enabled();
    if (timing) {
        XSYMV_HIP(timed_call_create(tc, timing, false));  // no merge step
    }
    Syr2Args<T> sa{A, xin, yin, plan->d_blocks, plan->d_strip_base, (long long)lda, alpha, n};
    XSYMV_HIP(launch_k(kern, plan->G, threads, stream, sa, tc.e0, tc.e1));
    if (timing) timing_push(tc);
    return 0;
}

// ------------------------------------------------------------------ xTRMV
template <class T>
struct TrmvKernelSet {
    int W, SW, G, NT, split;
    void (*k[2][3][2])(TrmvArgs<T>);  // [upper][0 'N', 1 'T', 2 'C'][unit]
    int R() const { return W * SW * 64 * Elem<T>::VEC; }
};

template <class T, bool UP, int W, int SW, int G, bool NT>
void fill_trmv(void (*k[3][2])(TrmvArgs<T>))
{
    constexpr bool cplx = std::is_same<T, cf32>::value || std::is_same<T, cf64>::value;
    k[0][0] = &trmv_strip<T, UP, 0, false, W, SW, G, NT, STRIP_CBUF>;
    k[0][1] = &trmv_strip<T, UP, 0, true, W, SW, G, NT, STRIP_CBUF>;
    k[1][0] = &trmv_strip<T, UP, 1, false, W, SW, G, NT, STRIP_CBUF>;
    k[1][1] = &trmv_strip<T, UP, 1, true, W, SW, G, NT, STRIP_CBUF>;
    if constexpr (cplx) {
        k[2][0] = &trmv_strip<T, UP, 2, false, W, SW, G, NT, STRIP_CBUF>;
        k[2][1] = &trmv_strip<T, UP, 2, true, W, SW, G, NT, STRIP_CBUF>;
    } else {  // real: T^H = T^T
        k[2][0] = k[1][0];
        k[2][1] = k[1][1];
    }
}

template <class T, int W, int SW, int G, bool NT, int SPLIT>
TrmvKernelSet<T> make_trmv()
{
    TrmvKernelSet<T> k{W, SW, G, NT ? 1 : 0, SPLIT, {}};
    fill_trmv<T, false, W, SW, G, NT>(k.k[0]);
    fill_trmv<T, true, W, SW, G, NT>(k.k[1]);
    return k;
}

template <class T> const std::vector<TrmvKernelSet<T>>& trmv_kernel_sets();
// Built-in xTRMV choice per element type: [upper][0 'N', 1 'T' or 'C'][size
// class of n: below 12288, below 20000, then larger].
struct TrmvDefaults {
    int idx[2][2][3];
};
template <class T> TrmvDefaults trmv_defaults();
int trmv_selected(int prec);  // -1: the built-in choice

inline int trmv_size_class(int n) { return n < 12288 ? 0 : n < 20000 ? 1 : 2; }

template <class T>
int trmv_pick(bool upper, int tr, int n)
{
    const int sel = trmv_selected(prec_code<T>());
    return sel >= 0 ? sel
                    : trmv_defaults<T>().idx[upper ? 1 : 0][tr != 0 ? 1 : 0][trmv_size_class(n)];
}
int check_trmv_args(char uplo, char trans, char diag, int n, const void* A, int lda,
                    const void* x, int incx, bool* upper, int* tr, bool* unit);

// Workspace of a TRMV call: [partials][x gathered]
template <class T>
size_t trmv_workspace_bytes(int tr, int nseg, int R, int NS, int n)
{
    const size_t part = tr == 0 ? (size_t)nseg * R : (size_t)NS * n;
    return align_up(part * sizeof(T)) + align_up((size_t)n * sizeof(T));
}

template <class T>
int trmv_run(char uplo, char trans, char diag, int n, const T* A, int lda, T* x, int incx,
             hipStream_t stream, int forced_idx)
{
    bool upper = false, unit = false;
    int tr = 0;
    int rc = check_trmv_args(uplo, trans, diag, n, A, lda, x, incx, &upper, &tr, &unit);
    if (rc) return rc;
    if (n == 0) return 0;
    const auto& ks = trmv_kernel_sets<T>()[forced_idx >= 0 ? forced_idx : trmv_pick<T>(upper, tr, n)];
    const int R = ks.R();
    const int threads = 64 * ks.W;
    auto kern = ks.k[upper ? 1 : 0][tr][unit ? 1 : 0];
    int dev = 0;
    XSYMV_HIP(hipGetDevice(&dev));
    DeviceState* ds = device_state(dev);
    std::lock_guard<std::mutex> lk(device_mutex(ds));
    int G = 0;
    rc = resident_blocks((const void*)kern, threads, &G);
    if (rc) return rc;
    const StripPlan* plan = nullptr;
    rc = get_strip_plan(ds, dev, upper, n, R, G, ks.split, stream, &plan);
    if (rc) return rc;
    void* ws = nullptr;
    rc = get_workspace(ds, stream, trmv_workspace_bytes<T>(tr, plan->nseg, R, plan->NS, n), &ws);
    if (rc) return rc;
    char* base = static_cast<char*>(ws);
    const size_t part_bytes = align_up((tr == 0 ? (size_t)plan->nseg * R : (size_t)plan->NS * n) *
                                       sizeof(T));
    T* part = reinterpret_cast<T*>(base);
    T* xg = reinterpret_cast<T*>(base + part_bytes);
    const long long kx = incx > 0 ? 0 : (long long)(1 - n) * incx;
    const T* xin = x;
    if (incx != 1) {
        symv_gather<T><<<blocks_for(n, 256), 256, 0, stream>>>(x, incx, kx, n, xg);
        XSYMV_HIP(hipGetLastError());
        xin = xg;
    }
    TimedCall tc{};
    const int timing = timing_enabled();
    if (timing) {
        XSYMV_HIP(timed_call_create(tc, timing));
    }
    TrmvArgs<T> ta{A, xin, part, part, plan->d_blocks, plan->d_strip_base, (long long)lda, n};
    XSYMV_HIP(launch_k(kern, plan->G, threads, stream, ta, tc.e0, tc.e1));
    TrmvMergeArgs<T> ma{part, plan->d_seg_base, xin, x, (long long)incx, kx, n, plan->NS, R,
                        upper ? 1 : 0, tr, unit ? 1 : 0};
    XSYMV_HIP(launch_k(&trmv_merge<T, MERGE_SPLIT>, blocks_for(n, 64), 64 * MERGE_SPLIT, stream,
                       ma, nullptr, tc.e2));
    if (timing) timing_push(tc);
    return 0;
}

template <class T>
size_t trmv_ws_bytes(char uplo, char trans, int n)
{
    const bool upper = uplo == 'U' || uplo == 'u';
    const int tr = (trans == 'N' || trans == 'n') ? 0 : 1;
    if (n <= 0) return 0;
    const auto& ks = trmv_kernel_sets<T>()[trmv_pick<T>(upper, tr, n)];
    size_t most = 0;
    for (int unit = 0; unit < 2; ++unit) {  // the larger of the two diagonal kinds
        int G = 0;
        if (resident_blocks((const void*)ks.k[upper ? 1 : 0][tr][unit], 64 * ks.W, &G))
            return (size_t)-1;
        std::vector<StripBlock> blocks;
        std::vector<int> sb, segb;
        int NS = 0;
        build_strip_plan_host(upper, n, ks.R(), G, ks.split, blocks, sb, segb, NS);
        most = std::max(most, trmv_workspace_bytes<T>(tr, segb[NS], ks.R(), NS, n));
    }
    return most;
}

// ------------------------------------------------- one shard's product
template <class T>
struct ShardKernelSet {
    int W, SW, G, NT, split;
    void (*k[2])(StripArgs<T>);  // lower, upper
    int R() const { return W * SW * 64 * Elem<T>::VEC; }
};

template <class T, int W, int SW, int G, bool NT, int SPLIT>
ShardKernelSet<T> make_shard()
{
    return ShardKernelSet<T>{W, SW, G, NT ? 1 : 0, SPLIT,
                             {&symv_strip<T, false, W, SW, G, NT, STRIP_CBUF, true>,
                              &symv_strip<T, true, W, SW, G, NT, STRIP_CBUF, true>}};
}

template <class T> const ShardKernelSet<T>& shard_kernels();
int check_shard_args(char uplo, int n, int panel, int nshards, int shard, const void* A, int lda,
                     const void* x, int incx, const void* p, bool* upper, int* ncol);
int check_combine_args(int n, int nshards, const void* P, int ldp, const void* y, int incy);

// Workspace of one shard's product: [rowpart nseg*R][colpart NS*ncol][x gathered, n]
template <class T>
size_t shard_workspace_bytes(int nseg, int R, int NS, int ncol, int n)
{
    return align_up((size_t)nseg * R * sizeof(T)) + align_up((size_t)NS * ncol * sizeof(T)) +
           align_up((size_t)n * sizeof(T));
}

// p := one shard's share of S*x (its own columns' stored elements in both
// roles, the diagonal once), contiguous; with no columns, p := 0.
template <class T>
int shard_run(char uplo, int n, int panel, int nshards, int shard, const T* A, int lda,
              const T* x, int incx, T* p, hipStream_t stream)
{
    bool upper = false;
    int ncol = 0;
    int rc = check_shard_args(uplo, n, panel, nshards, shard, A, lda, x, incx, p, &upper, &ncol);
    if (rc) return rc;
    if (n == 0) return 0;
    if (ncol == 0) {
        symv_scale<T><<<blocks_for(n, 256), 256, 0, stream>>>(p, 1, 0, n, tune_zero<T>(), 1);
        XSYMV_HIP(hipGetLastError());
        return 0;
    }
    const ShardKernelSet<T>& ks = shard_kernels<T>();
    const int R = ks.R();
    const int threads = 64 * ks.W;
    auto kern = ks.k[upper ? 1 : 0];
    int dev = 0;
    XSYMV_HIP(hipGetDevice(&dev));
    DeviceState* ds = device_state(dev);
    std::lock_guard<std::mutex> lk(device_mutex(ds));
    int G = 0;
    rc = resident_blocks((const void*)kern, threads, &G);
    if (rc) return rc;
    const StripPlan* plan = nullptr;
    rc = get_shard_plan(ds, upper, n, R, G, ks.split, panel, nshards, shard, stream, &plan);
    if (rc) return rc;
    void* ws = nullptr;
    rc = get_workspace(ds, stream, shard_workspace_bytes<T>(plan->nseg, R, plan->NS, ncol, n), &ws);
    if (rc) return rc;
    char* base = static_cast<char*>(ws);
    const size_t off_col = align_up((size_t)plan->nseg * R * sizeof(T));
    const size_t off_x = off_col + align_up((size_t)plan->NS * ncol * sizeof(T));
    T* rowpart = reinterpret_cast<T*>(base);
    T* colpart = reinterpret_cast<T*>(base + off_col);
    T* xg = reinterpret_cast<T*>(base + off_x);
    const T* xin = x;
    if (incx != 1) {
        const long long kx = incx > 0 ? 0 : (long long)(1 - n) * incx;
        symv_gather<T><<<blocks_for(n, 256), 256, 0, stream>>>(x, incx, kx, n, xg);
        XSYMV_HIP(hipGetLastError());
        xin = xg;
    }
    TimedCall tc{};
    const int timing = timing_enabled();
    if (timing) {
        XSYMV_HIP(timed_call_create(tc, timing));
    }
    StripArgs<T> sa{A, xin, rowpart, colpart, plan->d_blocks, plan->d_strip_base,
                    (long long)lda, n, plan->d_lcol, plan->d_gloc, plan->d_col0, ncol};
    XSYMV_HIP(launch_k(kern, plan->G, threads, stream, sa, tc.e0, tc.e1));
    StripMergeArgs<T> ma{rowpart, colpart, plan->d_seg_base, p, 1, 0, tune_one<T>(),
                         tune_zero<T>(), n, plan->NS, R, upper ? 1 : 0, 1, plan->d_gloc, ncol};
    XSYMV_HIP((launch_strip_merge<T, MERGE_SPLIT, true>(ma, n, stream, tc.e2,
                                                         plan->h_seg_base.data())));
    if (timing) timing_push(tc);
    return 0;
}

// y := beta*y + alpha*(P[0] + P[1] + ...), the partials summed in rank order.
template <class T>
int combine_run(int n, int nshards, T alpha, const T* P, int ldp, T beta, T* y, int incy,
                hipStream_t stream)
{
    int rc = check_combine_args(n, nshards, P, ldp, y, incy);
    if (rc) return rc;
    if (n == 0 || (host_is_zero(alpha) && host_is_one(beta))) return 0;
    const long long ky = incy > 0 ? 0 : (long long)(1 - n) * incy;
    const int beta_zero = host_is_zero(beta) ? 1 : 0;
    if (host_is_zero(alpha)) {
        symv_scale<T><<<blocks_for(n, 256), 256, 0, stream>>>(y, incy, ky, n, beta, beta_zero);
        XSYMV_HIP(hipGetLastError());
        return 0;
    }
    CombineArgs<T> ca{P, y, (long long)ldp, (long long)incy, ky, alpha, beta, n, nshards,
                      beta_zero};
    TimedCall tc{};
    const int timing = timing_enabled();
    if (timing) XSYMV_HIP(timed_call_create(tc, timing, false));  // one kernel
    XSYMV_HIP(launch_k(&symv_combine<T>, blocks_for(n, 256), 256, stream, ca, tc.e0, tc.e1));
    if (timing) timing_push(tc);
    return 0;
}

template <class T>
size_t shard_ws_bytes(char uplo, int n, int panel, int nshards, int shard)
{
    bool upper = false;
    int ncol = 0;
    if (check_shard_args(uplo, n, panel, nshards, shard, (const void*)1, std::max(1, n),
                         (const void*)1, 1, (const void*)1, &upper, &ncol))
        return (size_t)-1;
    if (n == 0 || ncol == 0) return 0;
    const ShardKernelSet<T>& ks = shard_kernels<T>();
    int G = 0;
    if (resident_blocks((const void*)ks.k[upper ? 1 : 0], 64 * ks.W, &G)) return (size_t)-1;
    std::vector<int> cols, col0;
    shard_columns_host(n, panel, nshards, shard, cols);
    std::vector<StripBlock> blocks;
    std::vector<int> sb, segb;
    int NS = 0;
    build_strip_plan_host(upper, n, ks.R(), G, ks.split, blocks, sb, segb, NS, &cols, &col0);
    return shard_workspace_bytes<T>(segb[NS], ks.R(), NS, ncol, n);
}

// ---------------------------------------------------------------- autotuner
// Deterministic test data for timing: a counter-based hash of the index
// mapped to [-1, 1) in every real word.
__device__ __forceinline__ double tune_value(unsigned long long i)
{
    unsigned long long z = i + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}
template <class T> __device__ T tune_elem(unsigned long long i);
template <> __device__ inline float tune_elem<float>(unsigned long long i) { return (float)tune_value(i); }
template <> __device__ inline double tune_elem<double>(unsigned long long i) { return tune_value(i); }
template <> __device__ inline cf32 tune_elem<cf32>(unsigned long long i)
{
    return {(float)tune_value(2 * i), (float)tune_value(2 * i + 1)};
}
template <> __device__ inline cf64 tune_elem<cf64>(unsigned long long i)
{
    return {tune_value(2 * i), tune_value(2 * i + 1)};
}
template <> __device__ inline ddreal tune_elem<ddreal>(unsigned long long i)
{
    const double h = tune_value(2 * i);
    return {h, h * tune_value(2 * i + 1) * 0x1p-53};
}

template <class T>
__global__ __launch_bounds__(256) void tune_fill(T* a, long long count, unsigned long long seed)
{
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < count;
         i += (long long)gridDim.x * 256)
        a[i] = tune_elem<T>(seed + (unsigned long long)i);
}

// Flush the caches (L2, MALL) between timed calls: write a 1 GiB buffer,
// then read it back, so that the caches hold clean lines of the buffer and
// the timed call pays no write-back of dirty ones.
static __global__ __launch_bounds__(256) void tune_flush(uint32_t* buf, long long words)
{
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < words;
         i += (long long)gridDim.x * 256)
        buf[i] = (uint32_t)i;
}

static __global__ __launch_bounds__(256) void tune_flush_read(uint32_t* buf, long long words)
{
    uint32_t acc = 0;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < words;
         i += (long long)gridDim.x * 256)
        acc ^= buf[i];
    // never true for what tune_flush wrote (values below 2^28, so their XOR
    // is too), but it keeps the loads from being dropped
    if (acc == 0xffffffffu) buf[0] = acc;
}

// Time every configuration of T for (uplo, n) on a matrix of leading
// dimension lda: `reps` calls each (after two warm-up calls), each preceded
// by a cache flush (1 GiB written and read back) when the matrix is smaller
// than 1 GiB; the configuration
// with the lowest median wins, ties going to the lower index.  ms[i]
// receives configuration i's median (up to max_cfg).
template <class T>
int autotune_impl(char uplo, int n, int lda_arg, int reps, hipStream_t stream, int* best_idx,
                  float* ms, int max_cfg)
{
    if (n <= 0 || reps <= 0 || lda_arg < n ||
        !(uplo == 'U' || uplo == 'u' || uplo == 'L' || uplo == 'l'))
        return -1;
    const long long lda = lda_arg;
    const size_t abytes = (size_t)lda * n * sizeof(T);
    T *A = nullptr, *x = nullptr, *y = nullptr;
    uint32_t* fl = nullptr;
    const long long flush_words = (1ll << 30) / 4;
    const bool flush = abytes < ((size_t)1 << 30);
    int rc = 0;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    const auto& sets = kernel_sets<T>();
    std::vector<float> med(sets.size(), 0.f);
    auto fail = [&](hipError_t e) { rc = ERR_HIP + (int)e; };
    hipError_t e;
    if ((e = hipMalloc((void**)&A, abytes)) != hipSuccess) { fail(e); goto done; }
    if ((e = hipMalloc((void**)&x, n * sizeof(T))) != hipSuccess) { fail(e); goto done; }
    if ((e = hipMalloc((void**)&y, n * sizeof(T))) != hipSuccess) { fail(e); goto done; }
    if (flush && (e = hipMalloc((void**)&fl, flush_words * 4)) != hipSuccess) { fail(e); goto done; }
    if ((e = hipEventCreate(&e0)) != hipSuccess || (e = hipEventCreate(&e1)) != hipSuccess) {
        fail(e);
        goto done;
    }
    tune_fill<T><<<4096, 256, 0, stream>>>(A, lda * n, 1);
    tune_fill<T><<<64, 256, 0, stream>>>(x, n, 1ull << 40);
    tune_fill<T><<<64, 256, 0, stream>>>(y, n, 1ull << 41);
    for (size_t ci = 0; ci < sets.size(); ++ci) {
        std::vector<float> t;
        for (int r = 0; r < reps + 2 && rc == 0; ++r) {
            if (flush) {
                tune_flush<<<2048, 256, 0, stream>>>(fl, flush_words);
                tune_flush_read<<<2048, 256, 0, stream>>>(fl, flush_words);
            }
            if ((e = hipEventRecord(e0, stream)) != hipSuccess) { fail(e); break; }
            // alpha = 1, beta = 0: y is overwritten, never grows
            rc = symv_run<T>(uplo, n, tune_one<T>(), A, (int)lda, x, 1, tune_zero<T>(), y, 1,
                             stream, (int)ci);
            if (rc) break;
            if ((e = hipEventRecord(e1, stream)) != hipSuccess) { fail(e); break; }
            if ((e = hipEventSynchronize(e1)) != hipSuccess) { fail(e); break; }
            float v = 0.f;
            if ((e = hipEventElapsedTime(&v, e0, e1)) != hipSuccess) { fail(e); break; }
            if (r >= 2) t.push_back(v);
        }
        if (rc) goto done;
        std::sort(t.begin(), t.end());
        med[ci] = t[t.size() / 2];
    }
    {
        size_t best = 0;
        for (size_t ci = 1; ci < sets.size(); ++ci)
            if (med[ci] < med[best]) best = ci;
        if (best_idx) *best_idx = (int)best;
        for (size_t ci = 0; ci < sets.size() && (int)ci < max_cfg; ++ci)
            if (ms) ms[ci] = med[ci];
    }
done:
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    (void)hipStreamSynchronize(stream);
    if (A) (void)hipFree(A);
    if (x) (void)hipFree(x);
    if (y) (void)hipFree(y);
    if (fl) (void)hipFree(fl);
    return rc;
}

template <class T>
size_t ws_bytes_config(bool upper, int n, int idx);

template <class T>
size_t ws_bytes(char uplo, int n)
{
    if (n <= 0) return 0;
    const bool upper = (uplo == 'U' || uplo == 'u');
    // the leading dimension is not known here: the larger need of the two
    // stride classes' choices
    const int c0 = pick_config(prec_code<T>(), upper, n, 0);
    const int c1 = pick_config(prec_code<T>(), upper, n, 1);
    if (c0 != c1) return std::max(ws_bytes_config<T>(upper, n, c0), ws_bytes_config<T>(upper, n, c1));
    return ws_bytes_config<T>(upper, n, c0);
}

template <class T>
size_t ws_bytes_config(bool upper, int n, int idx)
{
    const KernelSet<T>& ks = kernel_sets<T>()[idx];
    const ConfigInfo& ci = ks.info;
    if (ci.strip()) {
        int G = 0;
        if (resident_blocks((const void*)(upper ? ks.strip_upper : ks.strip_lower), 64 * ci.W,
                            &G))
            return (size_t)-1;
        std::vector<StripBlock> blocks;
        std::vector<int> sb, segb;
        int NS = 0;
        build_strip_plan_host(upper, n, ci.R(), G, ci.RUNS - 4, blocks, sb, segb, NS);
        return strip_workspace_bytes<T>(segb[NS], ci.R(), NS, n);
    }
    std::vector<TileDesc> tiles;
    std::vector<int> sb;
    int P = 0;
    build_plan_host(upper, n, ci.NB(), ci.R(), tiles, sb, P);
    return workspace_bytes_for<T>(P, n, sb[P], ci.NB());
}

}  // namespace xsymv
