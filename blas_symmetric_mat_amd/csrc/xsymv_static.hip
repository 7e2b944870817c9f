// xsymv_static.hip -- SSYMV for callers that cannot allocate device memory.
//
// The same product as xsymv_s (the CUDA-xSYMV report's eq.(1), §1), with the
// same configuration choice, kernels and work split, so the same bytes; only
// the device memory beyond A, x and y differs.  xsymv_s keeps a workspace per
// stream (hipMalloc on first use) and cached work splits (hipMalloc and
// pinned host memory); this entry point places both in `scratch`, one array
// per GPU in the code object's device memory:
//
//   [work split: StripBlock per workgroup, strip_base[NS+1], seg_base[NS+1]]
//   [rowpart nseg*R][colpart NS*n][x gathered, n (non-unit incx only)]
//
// Nothing in it has to start at zero: the streaming kernel writes every row
// and column partial that the merge reads, in the same call.  The work split
// is written only when the shape (triangle, n, configuration) differs from
// the one the array holds, by a copy from host memory that the call waits
// for; a call of the shape the array already holds enqueues kernels only.
//
// Calls on one GPU share the array: calls on one stream are ordered, calls
// that overlap in time (other streams, other threads) race on it.
#include "xsymv_host.hpp"

#include <array>
#include <cstring>

namespace xsymv {
namespace {

// The array.  In host code `scratch` names a host-side stand-in: the device
// address comes from hipGetSymbolAddress, per device, and only that address
// is ever handed to a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[XSYMV_STATIC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;

struct StaticState {
    char* base = nullptr;  // device address of `scratch` on this device
    bool have_split = false;
    // shape of the work split the array holds
    int upper = 0, n = 0, R = 0, G = 0, split = 0;
    int NS = 0, nblocks = 0, nseg = 0;
    std::vector<int> seg;  // host copy of seg_base (passed to the merge as arguments)
};

std::mutex g_static_mu;
std::array<StaticState, MAX_DEVICES> g_static;

// Byte layout of the array for a split of nblocks workgroups, NS strips and
// nseg segments; returns the bytes needed.
template <class T>
size_t static_layout(int nblocks, int NS, int nseg, int R, int n, bool gather, size_t* o_sb,
                     size_t* o_seg, size_t* o_row, size_t* o_col, size_t* o_x)
{
    *o_sb = align_up((size_t)nblocks * sizeof(StripBlock));
    *o_seg = *o_sb + align_up((size_t)(NS + 1) * sizeof(int));
    *o_row = *o_seg + align_up((size_t)(NS + 1) * sizeof(int));
    *o_col = *o_row + align_up((size_t)nseg * R * sizeof(T));
    *o_x = *o_col + align_up((size_t)NS * n * sizeof(T));
    return *o_x + (gather ? align_up((size_t)n * sizeof(T)) : 0);
}

template <class T>
int symv_static(char uplo, int n, T alpha, const T* A, int lda, const T* x, int incx, T beta,
                T* y, int incy, hipStream_t stream)
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
    const int idx = pick_config(prec_code<T>(), upper, n, stride_class(lda, sizeof(T)));
    const KernelSet<T>& ks = kernel_sets<T>()[idx];
    if (!ks.info.strip()) return ERR_STATIC_CONFIG;
    const int R = ks.info.R();
    const int threads = 64 * ks.info.W;
    const int split = ks.info.RUNS - 4;
    auto kern = upper ? ks.strip_upper : ks.strip_lower;

    int dev = 0;
    XSYMV_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= MAX_DEVICES) return ERR_STATIC_DEVICE;
    int G = 0;
    rc = resident_blocks((const void*)kern, threads, &G);
    if (rc) return rc;

    std::lock_guard<std::mutex> lk(g_static_mu);
    StaticState& st = g_static[dev];
    if (st.base == nullptr) {
        // once per device, with that device current
        void* p = nullptr;
        XSYMV_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        st.base = static_cast<char*>(p);
    }
    const bool gather = incx != 1;
    size_t o_sb, o_seg, o_row, o_col, o_x;
    const bool same = st.have_split && st.upper == (upper ? 1 : 0) && st.n == n && st.R == R &&
                      st.G == G && st.split == split;
    if (!same) {
        std::vector<StripBlock> blocks;
        std::vector<int> sb, segb;
        int NS = 0, g = G;
        build_strip_plan_host(upper, n, R, g, split, blocks, sb, segb, NS);
        const int nblocks = (int)blocks.size();
        const size_t need = static_layout<T>(nblocks, NS, segb[NS], R, n, gather, &o_sb, &o_seg,
                                             &o_row, &o_col, &o_x);
        if (need > XSYMV_STATIC_SCRATCH_BYTES) return ERR_STATIC_SIZE;  // nothing enqueued
        std::vector<char> h(o_row, 0);
        std::memcpy(h.data(), blocks.data(), blocks.size() * sizeof(StripBlock));
        std::memcpy(h.data() + o_sb, sb.data(), sb.size() * sizeof(int));
        std::memcpy(h.data() + o_seg, segb.data(), segb.size() * sizeof(int));
        // the array's old split may still be read by work queued on `stream`:
        // the copy is ordered after it, and the call waits for the copy so
        // that the host buffer can go
        st.have_split = false;
        XSYMV_HIP(hipMemcpyAsync(st.base, h.data(), o_row, hipMemcpyHostToDevice, stream));
        XSYMV_HIP(hipStreamSynchronize(stream));
        st.have_split = true;
        st.upper = upper ? 1 : 0;
        st.n = n;
        st.R = R;
        st.G = G;
        st.split = split;
        st.NS = NS;
        st.nblocks = nblocks;
        st.nseg = segb[NS];
        st.seg = segb;
    } else {
        const size_t need = static_layout<T>(st.nblocks, st.NS, st.nseg, R, n, gather, &o_sb,
                                             &o_seg, &o_row, &o_col, &o_x);
        if (need > XSYMV_STATIC_SCRATCH_BYTES) return ERR_STATIC_SIZE;  // (the gathered x)
    }
    char* base = st.base;
    const StripBlock* d_blocks = reinterpret_cast<const StripBlock*>(base);
    const int* d_strip_base = reinterpret_cast<const int*>(base + o_sb);
    const int* d_seg_base = reinterpret_cast<const int*>(base + o_seg);
    T* rowpart = reinterpret_cast<T*>(base + o_row);
    T* colpart = reinterpret_cast<T*>(base + o_col);
    const T* xin = x;
    if (gather) {
        T* xg = reinterpret_cast<T*>(base + o_x);
        symv_gather<T><<<blocks_for(n, 256), 256, 0, stream>>>(x, incx, kx, n, xg);
        XSYMV_HIP(hipGetLastError());
        xin = xg;
    }
    StripArgs<T> sa{A, xin, rowpart, colpart, d_blocks, d_strip_base, (long long)lda, n};
    kern<<<st.nblocks, threads, 0, stream>>>(sa);
    XSYMV_HIP(hipGetLastError());
    StripMergeArgs<T> ma{rowpart, colpart, d_seg_base, y, (long long)incy, ky, alpha, beta,
                         n, st.NS, R, upper ? 1 : 0, beta_zero};
    XSYMV_HIP((launch_strip_merge<T, MERGE_SPLIT>(ma, n, stream, nullptr, st.seg.data())));
    return 0;
}

}  // namespace
}  // namespace xsymv

extern "C" int xsymv_s_noalloc(char uplo, int n, float alpha, const float* A, int lda,
                               const float* x, int incx, float beta, float* y, int incy,
                               void* stream)
{
    return xsymv::symv_static<float>(uplo, n, alpha, A, lda, x, incx, beta, y, incy,
                                     (hipStream_t)stream);
}
