// xsymv_host.hip -- state shared by all precisions of libxsymv (selection
// rules, tile plans, per-stream workspaces, timing) and the precision-generic
// C ABI calls of include/xsymv.h.
#include "xsymv_host.hpp"

#include <algorithm>
#include <atomic>
#include <cctype>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

namespace xsymv {

namespace {
struct Rule {
    int n_lo, n_hi, idx;
};
std::mutex g_rules_mu;
std::vector<Rule> g_rules[5][2];

std::mutex g_time_mu;
int g_timing = 0;  // 0 off, 1 main kernel and merge, 2 whole call
std::vector<TimedCall> g_timed;

std::mutex g_dev_mu;
}  // namespace

using PlanKey = std::tuple<int, int, int, int, int>;  // upper, n, NB, R, device

using StripKey = std::tuple<int, int, int, int, int>;  // upper, n, R, G, split
// upper, n, R, G, split, panel, nshards, shard
using ShardKey = std::tuple<int, int, int, int, int, int, int, int>;

struct DeviceState {
    std::mutex mu;
    std::map<PlanKey, std::unique_ptr<Plan>> plans;
    std::map<StripKey, std::unique_ptr<StripPlan>> strip_plans;
    std::map<ShardKey, std::unique_ptr<StripPlan>> shard_plans;
    std::map<std::tuple<int, int, int, int>, std::unique_ptr<StripPlan>> gemv_plans;  // m, n, R, G
    std::map<hipStream_t, Workspace> workspaces;
    // (kernel, threads) -> blocks.  Guarded by its own lock: size queries
    // reach it without `mu`, product calls with `mu` held.
    std::mutex resident_mu;
    std::map<std::pair<const void*, int>, int> resident;
};

namespace {
std::map<int, std::unique_ptr<DeviceState>> g_dev;
}


void build_plan_host(bool upper, int n, int NB, int R, std::vector<TileDesc>& tiles,
                     std::vector<int>& slot_base, int& P)
{
    P = (n + NB - 1) / NB;
    std::vector<TileDesc> full, other;
    slot_base.assign(P + 1, 0);
    int slot = 0;
    for (int p = 0; p < P; ++p) {
        const int c0 = p * NB;
        const int cend = std::min(n, c0 + NB);
        const bool ragged_cols = (cend - c0) != NB;
        slot_base[p] = slot;
        other.push_back(TileDesc{p, c0, cend, (slot++ << 2) | TILE_DIAG});
        const int lo = upper ? 0 : cend;
        const int hi = upper ? c0 : n;
        for (int r0 = lo; r0 < hi; r0 += R) {
            const int r1 = std::min(hi, r0 + R);
            const bool rag = ragged_cols || (r1 - r0) != R;
            TileDesc t{p, r0, r1, (slot++ << 2) | (rag ? TILE_RAGGED : TILE_FULL)};
            (rag ? other : full).push_back(t);
        }
    }
    slot_base[P] = slot;
    // the short diagonal and ragged tiles first, so that their latency
    // overlaps the streaming of the full tiles
    tiles = other;
    tiles.insert(tiles.end(), full.begin(), full.end());
}

void build_strip_plan_host(bool upper, int n, int R, int G, int split,
                           std::vector<StripBlock>& blocks, std::vector<int>& strip_base,
                           std::vector<int>& seg_base, int& NS, const std::vector<int>* lcol,
                           std::vector<int>* col0)
{
    NS = (n + R - 1) / R;
    strip_base.assign(NS + 1, 0);
    // first (local) column of each strip's sequence; global = local unless
    // the columns are a shard's
    std::vector<int> first(NS, 0);
    for (int i = 0; i < NS; ++i) {
        int width, c0;
        if (lcol == nullptr) {
            width = upper ? n - i * R : std::min(n, (i + 1) * R);
            c0 = upper ? i * R : 0;
        } else {
            // L: local columns with global index < (i+1)R; U: those >= iR
            const int bound = upper ? i * R : std::min(n, (i + 1) * R);
            const int below = (int)(std::lower_bound(lcol->begin(), lcol->end(), bound) -
                                    lcol->begin());
            width = upper ? (int)lcol->size() - below : below;
            c0 = upper ? below : 0;
        }
        first[i] = c0;
        strip_base[i + 1] = strip_base[i] + width;
    }
    if (col0) *col0 = first;
    const long long total_pos = strip_base[NS];
    // Cost of one column of a strip, plus a fixed per-column share OVH for
    // the reductions.  A workgroup's time per column is set mostly by its
    // waves' per-column latency, not by how many of the column's rows are
    // stored, so
    //   split 0: the strip's height R per column, doubled in the diagonal
    //            triangle (the wave holding the diagonal takes element loads
    //            there, up to VEC of them per 16 bytes);
    //   split 1: the stored rows of the column plus R (suits element types of
    //            one or two elements per 16 bytes, whose band costs less);
    //   split 2: R per column, band or not (suits the double-double type,
    //            whose arithmetic, done for every row of a wave whether stored
    //            or not, sets the time of a band column as of any other).
    const long long OVH = 16;
    std::vector<long long> prefix(total_pos + 1, 0);
    long long pos = 0;
    for (int i = 0; i < NS; ++i) {
        const int rs0 = i * R, rs1 = std::min(n, rs0 + R), rows = rs1 - rs0;
        for (int t = 0; t < strip_base[i + 1] - strip_base[i]; ++t, ++pos) {
            const int j = lcol ? (*lcol)[first[i] + t] : first[i] + t;  // global column
            const bool tri = upper ? (j < rs1) : (j >= rs0);
            long long c;
            if (split == 0) {
                c = tri ? 2ll * rows : rows;
            } else if (split == 2) {
                c = rows;
            } else {
                const long long stored = !tri ? rows : (upper ? (j - rs0 + 1) : (rs1 - j));
                c = stored + R;
            }
            prefix[pos + 1] = prefix[pos] + c + OVH;
        }
    }
    const long long C = prefix[total_pos];
    G = std::max(1, (int)std::min<long long>(G, total_pos));
    blocks.assign(G, StripBlock{});
    std::vector<long long> bound(G + 1, 0);
    bound[G] = total_pos;
    for (int b = 1; b < G; ++b) {
        // first position whose prefix cost reaches b*C/G
        const long long target = (C * (long long)b) / G;
        bound[b] = std::lower_bound(prefix.begin(), prefix.end(), target) - prefix.begin();
        bound[b] = std::max(bound[b], bound[b - 1]);
        bound[b] = std::min(bound[b], total_pos);
    }
    seg_base.assign(NS + 1, 0);
    int slot = 0;
    int strip = 0;
    std::vector<int> first_slot(NS, -1);
    for (int b = 0; b < G; ++b) {
        const int u0 = (int)bound[b], u1 = (int)bound[b + 1];
        while (strip < NS - 1 && strip_base[strip + 1] <= u0) ++strip;
        blocks[b] = StripBlock{u0, u1, slot, strip, strip_base[strip], strip_base[strip + 1],
                               first[strip], 0};
        int u = u0, st = strip;
        while (u < u1) {
            if (first_slot[st] < 0) first_slot[st] = slot;
            u = std::min(u1, strip_base[st + 1]);
            ++slot;
            ++st;
        }
    }
    // A strip holding none of the sequence (a shard's strip with none of its
    // columns) has no segment unless a range steps through it: its first
    // slot is then the next strip's, so that it counts zero row partials.
    seg_base[NS] = slot;
    for (int i = NS - 1; i >= 0; --i) seg_base[i] = first_slot[i] >= 0 ? first_slot[i] : seg_base[i + 1];
}

DeviceState* device_state(int dev)
{
    std::lock_guard<std::mutex> lk(g_dev_mu);
    auto& p = g_dev[dev];
    if (!p) p.reset(new DeviceState());
    return p.get();
}

std::mutex& device_mutex(DeviceState* ds) { return ds->mu; }

int get_plan(DeviceState* ds, int dev, bool upper, int n, int NB, int R, hipStream_t stream,
             const Plan** out)
{
    PlanKey key{upper ? 1 : 0, n, NB, R, dev};
    auto it = ds->plans.find(key);
    if (it != ds->plans.end()) {
        *out = it->second.get();
        return 0;
    }
    std::vector<TileDesc> tiles;
    std::vector<int> slot_base;
    int P = 0;
    build_plan_host(upper, n, NB, R, tiles, slot_base, P);
    std::unique_ptr<Plan> plan(new Plan());
    plan->P = P;
    plan->NB = NB;
    plan->ntiles = (int)tiles.size();
    plan->nslots = slot_base[P];
    const size_t tb = tiles.size() * sizeof(TileDesc);
    const size_t sb = slot_base.size() * sizeof(int);
    XSYMV_HIP(hipHostMalloc((void**)&plan->h_tiles, tb, hipHostMallocDefault));
    XSYMV_HIP(hipHostMalloc((void**)&plan->h_slot_base, sb, hipHostMallocDefault));
    std::copy(tiles.begin(), tiles.end(), plan->h_tiles);
    std::copy(slot_base.begin(), slot_base.end(), plan->h_slot_base);
    XSYMV_HIP(hipMalloc((void**)&plan->d_tiles, tb));
    XSYMV_HIP(hipMalloc((void**)&plan->d_slot_base, sb));
    XSYMV_HIP(hipMemcpyAsync(plan->d_tiles, plan->h_tiles, tb, hipMemcpyHostToDevice, stream));
    XSYMV_HIP(hipMemcpyAsync(plan->d_slot_base, plan->h_slot_base, sb, hipMemcpyHostToDevice,
                             stream));
    // A plan may later be used from other streams: finish the upload now.
    XSYMV_HIP(hipStreamSynchronize(stream));
    *out = plan.get();
    ds->plans[key] = std::move(plan);
    return 0;
}

int resident_blocks(const void* kernel, int threads, int* out)
{
    int dev = 0;
    XSYMV_HIP(hipGetDevice(&dev));
    DeviceState* ds = device_state(dev);
    auto key = std::make_pair(kernel, threads);
    std::lock_guard<std::mutex> lk(ds->resident_mu);
    auto it = ds->resident.find(key);
    if (it != ds->resident.end()) {
        *out = it->second;
        return 0;
    }
    int per_cu = 0, cus = 0;
    XSYMV_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0));
    XSYMV_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    *out = std::max(1, per_cu) * std::max(1, cus);
    ds->resident[key] = *out;
    return 0;
}

void build_gemv_plan_host(int m, int n, int R, int G, std::vector<StripBlock>& blocks,
                          std::vector<int>& seg_base, int& NS)
{
    NS = (m + R - 1) / R;
    const long long total = (long long)NS * n;
    const long long OVH = 16;
    // cost of one column of strip i: its rows + OVH; prefix over strips
    auto cost_before = [&](long long pos) {  // cost of positions [0, pos)
        const long long full = pos / n, rem = pos % n;
        long long c = 0;
        const long long rows_full = (long long)R + OVH;
        const long long last_rows = (long long)(m - (NS - 1) * R) + OVH;
        if (full >= NS) return (NS - 1) * n * rows_full + n * last_rows;
        c = full * n * rows_full;
        c += rem * (full == NS - 1 ? last_rows : rows_full);
        return c;
    };
    const long long C = cost_before(total);
    G = std::max(1, (int)std::min<long long>(G, total));
    blocks.assign(G, StripBlock{});
    std::vector<long long> bound(G + 1, 0);
    bound[G] = total;
    for (int b = 1; b < G; ++b) {
        const long long target = (C * (long long)b) / G;
        long long lo = bound[b - 1], hi = total;  // first pos with cost_before >= target
        while (lo < hi) {
            const long long mid = (lo + hi) / 2;
            if (cost_before(mid) < target)
                lo = mid + 1;
            else
                hi = mid;
        }
        bound[b] = lo;
    }
    seg_base.assign(NS + 1, 0);
    std::vector<int> first_slot(NS, -1);
    int slot = 0;
    for (int b = 0; b < G; ++b) {
        const int u0 = (int)bound[b], u1 = (int)bound[b + 1];
        const int strip = std::min(NS - 1, u0 / std::max(n, 1));
        blocks[b] = StripBlock{u0, u1, slot, strip, strip * n, (strip + 1) * n, 0, 0};
        int u = u0, st = strip;
        while (u < u1) {
            if (first_slot[st] < 0) first_slot[st] = slot;
            u = std::min(u1, (st + 1) * n);
            ++slot;
            ++st;
        }
    }
    // a strip none of whose positions is in a non-empty range cannot occur
    // (every position belongs to one range); keep seg_base monotone anyway
    for (int i = 0; i < NS; ++i) seg_base[i] = first_slot[i] < 0 ? slot : first_slot[i];
    seg_base[NS] = slot;
}

int get_gemv_plan(DeviceState* ds, int m, int n, int R, int G, hipStream_t stream,
                  const StripPlan** out)
{
    auto key = std::make_tuple(m, n, R, G);
    auto it = ds->gemv_plans.find(key);
    if (it != ds->gemv_plans.end()) {
        *out = it->second.get();
        return 0;
    }
    std::vector<StripBlock> blocks;
    std::vector<int> segb;
    int NS = 0;
    build_gemv_plan_host(m, n, R, G, blocks, segb, NS);
    std::unique_ptr<StripPlan> plan(new StripPlan());
    plan->NS = NS;
    plan->G = (int)blocks.size();
    plan->nseg = segb[NS];
    plan->R = R;
    plan->h_seg_base = segb;
    const size_t bb = blocks.size() * sizeof(StripBlock);
    const size_t ib = segb.size() * sizeof(int);
    char* h = nullptr;
    XSYMV_HIP(hipHostMalloc((void**)&h, bb + ib, hipHostMallocDefault));
    plan->h_pinned = h;
    std::copy(blocks.begin(), blocks.end(), reinterpret_cast<StripBlock*>(h));
    std::copy(segb.begin(), segb.end(), reinterpret_cast<int*>(h + bb));
    char* d = nullptr;
    XSYMV_HIP(hipMalloc((void**)&d, bb + ib));
    XSYMV_HIP(hipMemcpyAsync(d, h, bb + ib, hipMemcpyHostToDevice, stream));
    XSYMV_HIP(hipStreamSynchronize(stream));
    plan->d_blocks = reinterpret_cast<StripBlock*>(d);
    plan->d_seg_base = reinterpret_cast<int*>(d + bb);
    *out = plan.get();
    ds->gemv_plans[key] = std::move(plan);
    return 0;
}

int check_gemv_args(char trans, int m, int n, const void* A, int lda, const void* x, int incx,
                    const void* y, int incy, int* tr)
{
    if (trans == 'N' || trans == 'n')
        *tr = 0;
    else if (trans == 'T' || trans == 't')
        *tr = 1;
    else if (trans == 'C' || trans == 'c')
        *tr = 2;
    else
        return -1;
    if (m < 0) return -2;
    if (n < 0) return -3;
    if (m > 0 && n > 0 && A == nullptr) return -5;
    if (lda < std::max(1, m)) return -6;
    if (m > 0 && n > 0 && x == nullptr) return -7;
    if (incx == 0) return -8;
    if (m > 0 && n > 0 && y == nullptr) return -10;
    if (incy == 0) return -11;
    return 0;
}

namespace {
std::atomic<int> g_gemv_idx[5] = {-1, -1, -1, -1, -1};
std::atomic<int> g_syr2_idx[5] = {-1, -1, -1, -1, -1};
std::atomic<int> g_trmv_idx[5] = {-1, -1, -1, -1, -1};
}

int gemv_selected(int prec) { return g_gemv_idx[prec].load(); }
int syr2_selected(int prec) { return g_syr2_idx[prec].load(); }
int trmv_selected(int prec) { return g_trmv_idx[prec].load(); }

int check_trmv_args(char uplo, char trans, char diag, int n, const void* A, int lda,
                    const void* x, int incx, bool* upper, int* tr, bool* unit)
{
    if (uplo == 'U' || uplo == 'u')
        *upper = true;
    else if (uplo == 'L' || uplo == 'l')
        *upper = false;
    else
        return -1;
    if (trans == 'N' || trans == 'n')
        *tr = 0;
    else if (trans == 'T' || trans == 't')
        *tr = 1;
    else if (trans == 'C' || trans == 'c')
        *tr = 2;
    else
        return -2;
    if (diag == 'U' || diag == 'u')
        *unit = true;
    else if (diag == 'N' || diag == 'n')
        *unit = false;
    else
        return -3;
    if (n < 0) return -4;
    if (n > 0 && A == nullptr) return -5;
    if (lda < std::max(1, n)) return -6;
    if (n > 0 && x == nullptr) return -7;
    if (incx == 0) return -8;
    return 0;
}

int check_syr2_args(char uplo, int n, const void* x, int incx, const void* y, int incy,
                    const void* A, int lda, bool* upper)
{
    if (uplo == 'U' || uplo == 'u')
        *upper = true;
    else if (uplo == 'L' || uplo == 'l')
        *upper = false;
    else
        return -1;
    if (n < 0) return -2;
    if (n > 0 && x == nullptr) return -4;
    if (incx == 0) return -5;
    if (n > 0 && y == nullptr) return -6;
    if (incy == 0) return -7;
    if (n > 0 && A == nullptr) return -8;
    if (lda < std::max(1, n)) return -9;
    return 0;
}

int shard_owner(int panel_index, int nshards)
{
    const int round = panel_index / nshards, pos = panel_index % nshards;
    return (round & 1) ? nshards - 1 - pos : pos;
}

void shard_columns_host(int n, int panel, int nshards, int shard, std::vector<int>& cols)
{
    cols.clear();
    const int npanels = (n + panel - 1) / panel;
    for (int q = 0; q < npanels; ++q) {
        if (shard_owner(q, nshards) != shard) continue;
        const int c1 = std::min(n, (q + 1) * panel);
        for (int c = q * panel; c < c1; ++c) cols.push_back(c);
    }
}

int shard_column_count(int n, int panel, int nshards, int shard)
{
    int count = 0;
    const int npanels = (n + panel - 1) / panel;
    for (int q = 0; q < npanels; ++q)
        if (shard_owner(q, nshards) == shard) count += std::min(n, (q + 1) * panel) - q * panel;
    return count;
}

int check_shard_args(char uplo, int n, int panel, int nshards, int shard, const void* A, int lda,
                     const void* x, int incx, const void* p, bool* upper, int* ncol)
{
    if (uplo == 'U' || uplo == 'u')
        *upper = true;
    else if (uplo == 'L' || uplo == 'l')
        *upper = false;
    else
        return -1;
    if (n < 0) return -2;
    if (panel <= 0) return -3;
    if (nshards <= 0) return -4;
    if (shard < 0 || shard >= nshards) return -5;
    *ncol = shard_column_count(n, panel, nshards, shard);
    if (*ncol > 0 && A == nullptr) return -6;
    if (lda < std::max(1, n)) return -7;
    if (n > 0 && x == nullptr) return -8;
    if (incx == 0) return -9;
    if (n > 0 && p == nullptr) return -10;
    return 0;
}

int check_combine_args(int n, int nshards, const void* P, int ldp, const void* y, int incy)
{
    if (n < 0) return -1;
    if (nshards <= 0) return -2;
    if (n > 0 && P == nullptr) return -4;
    if (ldp < std::max(1, n)) return -5;
    if (n > 0 && y == nullptr) return -7;
    if (incy == 0) return -8;
    return 0;
}

int get_shard_plan(DeviceState* ds, bool upper, int n, int R, int G, int split, int panel,
                   int nshards, int shard, hipStream_t stream, const StripPlan** out)
{
    ShardKey key{upper ? 1 : 0, n, R, G, split, panel, nshards, shard};
    auto it = ds->shard_plans.find(key);
    if (it != ds->shard_plans.end()) {
        *out = it->second.get();
        return 0;
    }
    std::vector<int> cols, col0;
    shard_columns_host(n, panel, nshards, shard, cols);
    std::vector<int> gloc(n, -1);
    for (size_t l = 0; l < cols.size(); ++l) gloc[cols[l]] = (int)l;
    std::vector<StripBlock> blocks;
    std::vector<int> sb, segb;
    int NS = 0;
    int g = G;
    build_strip_plan_host(upper, n, R, g, split, blocks, sb, segb, NS, &cols, &col0);
    std::unique_ptr<StripPlan> plan(new StripPlan());
    plan->NS = NS;
    plan->G = (int)blocks.size();
    plan->nseg = segb[NS];
    plan->R = R;
    plan->h_seg_base = segb;
    plan->ncol = (int)cols.size();
    // one upload: blocks, strip_base, seg_base, col0, lcol, gloc
    const size_t bb = blocks.size() * sizeof(StripBlock);
    const size_t ib = sb.size() * sizeof(int);
    const size_t cb = col0.size() * sizeof(int);
    const size_t lb = cols.size() * sizeof(int);
    const size_t gb = gloc.size() * sizeof(int);
    const size_t total = bb + 2 * ib + cb + lb + gb;
    char* h = nullptr;
    XSYMV_HIP(hipHostMalloc((void**)&h, total, hipHostMallocDefault));
    plan->h_pinned = h;
    size_t off = 0;
    std::copy(blocks.begin(), blocks.end(), reinterpret_cast<StripBlock*>(h + off));
    const size_t o_sb = off += bb;
    std::copy(sb.begin(), sb.end(), reinterpret_cast<int*>(h + off));
    const size_t o_seg = off += ib;
    std::copy(segb.begin(), segb.end(), reinterpret_cast<int*>(h + off));
    const size_t o_c0 = off += ib;
    std::copy(col0.begin(), col0.end(), reinterpret_cast<int*>(h + off));
    const size_t o_l = off += cb;
    std::copy(cols.begin(), cols.end(), reinterpret_cast<int*>(h + off));
    const size_t o_g = off += lb;
    std::copy(gloc.begin(), gloc.end(), reinterpret_cast<int*>(h + off));
    char* d = nullptr;
    XSYMV_HIP(hipMalloc((void**)&d, total));
    XSYMV_HIP(hipMemcpyAsync(d, h, total, hipMemcpyHostToDevice, stream));
    XSYMV_HIP(hipStreamSynchronize(stream));
    plan->d_blocks = reinterpret_cast<StripBlock*>(d);
    plan->d_strip_base = reinterpret_cast<int*>(d + o_sb);
    plan->d_seg_base = reinterpret_cast<int*>(d + o_seg);
    plan->d_col0 = reinterpret_cast<int*>(d + o_c0);
    plan->d_lcol = reinterpret_cast<int*>(d + o_l);
    plan->d_gloc = reinterpret_cast<int*>(d + o_g);
    *out = plan.get();
    ds->shard_plans[key] = std::move(plan);
    return 0;
}

int get_strip_plan(DeviceState* ds, int dev, bool upper, int n, int R, int G, int split,
                   hipStream_t stream, const StripPlan** out)
{
    (void)dev;
    StripKey key{upper ? 1 : 0, n, R, G, split};
    auto it = ds->strip_plans.find(key);
    if (it != ds->strip_plans.end()) {
        *out = it->second.get();
        return 0;
    }
    std::vector<StripBlock> blocks;
    std::vector<int> sb, segb;
    int NS = 0;
    int g = G;
    build_strip_plan_host(upper, n, R, g, split, blocks, sb, segb, NS);
    std::unique_ptr<StripPlan> plan(new StripPlan());
    plan->NS = NS;
    plan->G = (int)blocks.size();
    plan->nseg = segb[NS];
    plan->R = R;
    plan->h_seg_base = segb;
    const size_t bb = blocks.size() * sizeof(StripBlock);
    const size_t ib = sb.size() * sizeof(int);
    char* h = nullptr;
    XSYMV_HIP(hipHostMalloc((void**)&h, bb + 2 * ib, hipHostMallocDefault));
    plan->h_pinned = h;
    std::copy(blocks.begin(), blocks.end(), reinterpret_cast<StripBlock*>(h));
    std::copy(sb.begin(), sb.end(), reinterpret_cast<int*>(h + bb));
    std::copy(segb.begin(), segb.end(), reinterpret_cast<int*>(h + bb + ib));
    char* d = nullptr;
    XSYMV_HIP(hipMalloc((void**)&d, bb + 2 * ib));
    XSYMV_HIP(hipMemcpyAsync(d, h, bb + 2 * ib, hipMemcpyHostToDevice, stream));
    XSYMV_HIP(hipStreamSynchronize(stream));
    plan->d_blocks = reinterpret_cast<StripBlock*>(d);
    plan->d_strip_base = reinterpret_cast<int*>(d + bb);
    plan->d_seg_base = reinterpret_cast<int*>(d + bb + ib);
    *out = plan.get();
    ds->strip_plans[key] = std::move(plan);
    return 0;
}

int get_workspace(DeviceState* ds, hipStream_t stream, size_t bytes, void** out)
{
    auto& ws = ds->workspaces[stream];
    if (ws.bytes < bytes) {
        if (!ws.owned) return ERR_WORKSPACE;  // the caller's buffer is too small
        if (ws.ptr) {
            // the old buffer may still be in use by work queued on this stream
            XSYMV_HIP(hipStreamSynchronize(stream));
            XSYMV_HIP(hipFree(ws.ptr));
            ws.ptr = nullptr;
            ws.bytes = 0;
        }
        const size_t grown = std::max(bytes, (size_t)1 << 20);
        XSYMV_HIP(hipMalloc(&ws.ptr, grown));
        ws.bytes = grown;
    }
    *out = ws.ptr;
    return 0;
}

int timing_enabled()
{
    std::lock_guard<std::mutex> tl(g_time_mu);
    return g_timing;
}

void timing_push(const TimedCall& c)
{
    std::lock_guard<std::mutex> tl(g_time_mu);
    g_timed.push_back(c);
}

int check_args(char uplo, int n, const void* A, int lda, const void* x, int incx,
               const void* y, int incy, bool* upper)
{
    if (uplo == 'U' || uplo == 'u')
        *upper = true;
    else if (uplo == 'L' || uplo == 'l')
        *upper = false;
    else
        return -1;
    if (n < 0) return -2;
    if (n > 0 && A == nullptr) return -4;
    if (lda < std::max(1, n)) return -5;
    if (n > 0 && x == nullptr) return -6;
    if (incx == 0) return -7;
    if (n > 0 && y == nullptr) return -9;
    if (incy == 0) return -10;
    return 0;
}

namespace {
int num_configs(int prec)
{
    switch (prec) {
    case XSYMV_S: return (int)kernel_sets<float>().size();
    case XSYMV_D: return (int)kernel_sets<double>().size();
    case XSYMV_C: return (int)kernel_sets<cf32>().size();
    case XSYMV_Z: return (int)kernel_sets<cf64>().size();
    case XSYMV_W: return (int)kernel_sets<ddreal>().size();
    default: return -1;
    }
}

bool config_info(int prec, int idx, ConfigInfo* out)
{
    if (idx < 0 || idx >= num_configs(prec)) return false;
    switch (prec) {
    case XSYMV_S: *out = kernel_sets<float>()[idx].info; return true;
    case XSYMV_D: *out = kernel_sets<double>()[idx].info; return true;
    case XSYMV_C: *out = kernel_sets<cf32>()[idx].info; return true;
    case XSYMV_Z: *out = kernel_sets<cf64>()[idx].info; return true;
    case XSYMV_W: *out = kernel_sets<ddreal>()[idx].info; return true;
    default: return false;
    }
}
int find_config(int prec, int W, int CW, int S, int NT, int XL, int RUNS)
{
    ConfigInfo ci;
    for (int i = 0; i < num_configs(prec); ++i)
        if (config_info(prec, i, &ci) && ci.W == W && ci.CW == CW && ci.S == S && ci.NT == NT &&
            ci.XLDS == XL && ci.RUNS == RUNS)
            return i;
    return -1;
}

const char PREC_CHARS[5] = {'s', 'd', 'c', 'z', 'w'};

// Precision code of a precision letter, or -1.
int prec_of_char(char c)
{
    for (int p = 0; p < 5; ++p)
        if (PREC_CHARS[p] == c) return p;
    return -1;
}

}  // namespace

// Built-in selection rules measured on MI355X by the on-device autotuner over
// a grid of orders (the counterpart of the report's per-size rules, §3
// Table 3), for each stride class of the leading dimension (0: columns of
// whole 64-byte lines, measured with lda = n; 1: any other, measured with
// lda = n + 1).  Kernels are named by shape, so the table survives
// reordering of the configuration lists; rows whose shape is not compiled
// are ignored.
struct TunedRule {
    char prec, uplo;
    int n_lo, n_hi;
    int W, CW, S, NT, XLDS, RUNS;
    int cls;  // stride class (0 when omitted)
};
static const TunedRule TUNED_RULES[] = {
#include "xsymv_tuned.inc"
};

namespace {
std::once_flag g_builtin_once;
std::vector<Rule> g_builtin[5][2][2];  // [prec][upper][stride class]

void init_builtin_rules()
{
    for (const TunedRule& t : TUNED_RULES) {
        const int prec = prec_of_char(t.prec);
        if (prec < 0 || t.cls < 0 || t.cls > 1) continue;
        const int idx = find_config(prec, t.W, t.CW, t.S, t.NT, t.XLDS, t.RUNS);
        if (idx < 0) continue;
        g_builtin[prec][t.uplo == 'U' ? 1 : 0][t.cls].push_back(Rule{t.n_lo, t.n_hi, idx});
    }
}
}  // namespace

// The built-in rule of the stride class for n; class 1 falls back to class
// 0 where it has no rule; entry 0 when neither has one.
int builtin_config(int prec, bool upper, int n, int cls)
{
    std::call_once(g_builtin_once, init_builtin_rules);
    for (int c = cls; c >= 0; --c)
        for (const Rule& r : g_builtin[prec][upper ? 1 : 0][c])
            if (n >= r.n_lo && n <= r.n_hi) return r.idx;
    return 0;
}

// Caller rules first (the latest matching one, for every stride class; idx
// -1 defers to the built-in choice), then the built-in rules, then entry 0.
int pick_config(int prec, bool upper, int n, int cls)
{
    {
        std::lock_guard<std::mutex> lk(g_rules_mu);
        const auto& rs = g_rules[prec][upper ? 1 : 0];
        for (auto it = rs.rbegin(); it != rs.rend(); ++it)
            if (n >= it->n_lo && n <= it->n_hi) {
                if (it->idx >= 0) return it->idx;
                break;
            }
    }
    return builtin_config(prec, upper, n, cls);
}

namespace {


// A minimal reader for the rule files this library writes: a flat list of
// objects with string or integer values inside the "rules" array.
struct JsonRule {
    std::map<std::string, std::string> kv;
};

bool parse_rules(const std::string& text, std::vector<JsonRule>& out)
{
    size_t pos = text.find("\"rules\"");
    if (pos == std::string::npos) return false;
    pos = text.find('[', pos);
    if (pos == std::string::npos) return false;
    ++pos;
    auto skip_ws = [&]() {
        while (pos < text.size() && std::isspace((unsigned char)text[pos])) ++pos;
    };
    auto read_string = [&](std::string& v) -> bool {
        if (pos >= text.size() || text[pos] != '"') return false;
        size_t e = text.find('"', pos + 1);
        if (e == std::string::npos) return false;
        v = text.substr(pos + 1, e - pos - 1);
        pos = e + 1;
        return true;
    };
    for (;;) {
        skip_ws();
        if (pos >= text.size()) return false;
        if (text[pos] == ']') return true;
        if (text[pos] == ',') { ++pos; continue; }
        if (text[pos] != '{') return false;
        ++pos;
        JsonRule r;
        for (;;) {
            skip_ws();
            if (pos >= text.size()) return false;
            if (text[pos] == '}') { ++pos; break; }
            if (text[pos] == ',') { ++pos; continue; }
            std::string key, val;
            if (!read_string(key)) return false;
            skip_ws();
            if (pos >= text.size() || text[pos] != ':') return false;
            ++pos;
            skip_ws();
            if (pos < text.size() && text[pos] == '"') {
                if (!read_string(val)) return false;
            } else {
                size_t e = pos;
                while (e < text.size() && (std::isalnum((unsigned char)text[e]) ||
                                           text[e] == '-' || text[e] == '+' || text[e] == '.'))
                    ++e;
                if (e == pos) return false;
                val = text.substr(pos, e - pos);
                pos = e;
            }
            r.kv[key] = val;
        }
        out.push_back(r);
    }
}
}  // namespace

}  // namespace xsymv

using namespace xsymv;

// Plain streaming read, the reference point for "% of a measured
// stream-read peak": workgroup b reads its own contiguous chunk of `per`
// 16-byte vectors (non-temporal loads, U in flight per lane; `per` is a
// multiple of 256*U, so no load is guarded).
template <int U>
static __global__ __launch_bounds__(256) void read_probe(const xsymv::u32x4* __restrict__ a,
                                                           long long per, uint32_t* out)
{
    const xsymv::u32x4* __restrict__ p = a + (long long)blockIdx.x * per;
    uint32_t acc = 0;
    for (long long i = threadIdx.x; i < per; i += 256 * U) {
        xsymv::u32x4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) v[k] = __builtin_nontemporal_load(p + i + k * 256);
#pragma unroll
        for (int k = 0; k < U; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    // a store that depends on every load keeps them; it almost never happens
    // (a block-wide reduction here measurably lengthens the launch)
    if (acc == 0x9e3779b9u) out[blockIdx.x] = acc;
}

// The same read with every resident workgroup sweeping one address window:
// tile t (1024*U consecutive vectors) goes to workgroup t mod gridDim, so at
// any moment the device reads neighbouring tiles (measured faster on MI355X
// than a private chunk per workgroup).
template <int U>
static __global__ __launch_bounds__(1024) void read_probe_sweep(const xsymv::u32x4* __restrict__ a,
                                                                long long ntiles, uint32_t* out)
{
    uint32_t acc = 0;
    for (long long t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const xsymv::u32x4* __restrict__ p = a + t * (1024 * U) + threadIdx.x;
        xsymv::u32x4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) v[k] = __builtin_nontemporal_load(p + k * 1024);
#pragma unroll
        for (int k = 0; k < U; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    if (acc == 0x9e3779b9u) out[blockIdx.x] = acc;
}

// Plain read + write, the reference for the rank-2 update (which reads the
// stored triangle and writes it back): workgroup b copies its own chunk of
// `per` 16-byte vectors from src to dst, U vectors in flight per lane,
// non-temporal loads and stores.
template <int U>
static __global__ __launch_bounds__(256) void copy_probe(const xsymv::u32x4* __restrict__ src,
                                                         xsymv::u32x4* __restrict__ dst,
                                                         long long per)
{
    const xsymv::u32x4* __restrict__ p = src + (long long)blockIdx.x * per;
    xsymv::u32x4* __restrict__ q = dst + (long long)blockIdx.x * per;
    for (long long i = threadIdx.x; i < per; i += 256 * U) {
        xsymv::u32x4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) v[k] = __builtin_nontemporal_load(p + i + k * 256);
#pragma unroll
        for (int k = 0; k < U; ++k) __builtin_nontemporal_store(v[k], q + i + k * 256);
    }
}

static __global__ __launch_bounds__(256) void fill_probe(uint32_t* buf, long long words)
{
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < words;
         i += (long long)gridDim.x * 256)
        buf[i] = (uint32_t)(i * 2654435761u);
}

extern "C" {

size_t xsymv_workspace_bytes(int prec, char uplo, int n)
{
    switch (prec) {
    case XSYMV_S: return ws_bytes<float>(uplo, n);
    case XSYMV_D: return ws_bytes<double>(uplo, n);
    case XSYMV_C: return ws_bytes<cf32>(uplo, n);
    case XSYMV_Z: return ws_bytes<cf64>(uplo, n);
    case XSYMV_W: return ws_bytes<ddreal>(uplo, n);
    default: return (size_t)-1;
    }
}

int xsymv_read_bandwidth(size_t bytes, int reps, void* stream, float* gbps, float* best_gbps)
{
    if (bytes < ((size_t)64 << 20) || reps <= 0) return -1;
    const hipStream_t st = (hipStream_t)stream;
    const long long vecs = (long long)(bytes / 16);
    constexpr int MAXB = 32768;
    char* buf = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    int rc = 0;
    float best_med = 0.f, best_any = 0.f;
    auto fail = [&](hipError_t e) { rc = ERR_HIP + (int)e; };
    hipError_t e;
    if ((e = hipMalloc((void**)&buf, (size_t)vecs * 16 + MAXB * 4)) != hipSuccess)
        return ERR_HIP + (int)e;
    uint32_t* out = reinterpret_cast<uint32_t*>(buf + (size_t)vecs * 16);
    const auto* a = reinterpret_cast<const xsymv::u32x4*>(buf);
    fill_probe<<<4096, 256, 0, st>>>(reinterpret_cast<uint32_t*>(buf), vecs * 4);
    if ((e = hipGetLastError()) != hipSuccess) { fail(e); goto done; }
    if ((e = hipEventCreate(&e0)) != hipSuccess || (e = hipEventCreate(&e1)) != hipSuccess) {
        fail(e);
        goto done;
    }
    // a few layouts: a private chunk per workgroup (workgroups x loads in
    // flight per lane), then tiles swept by 1024-thread workgroups (grid x
    // loads in flight); the best median wins
    static const int chunk_blocks[3] = {2048, 8192, MAXB};
    for (int layout = 0; layout < 10; ++layout) {
        const bool sweep = layout >= 6;
        const int blocks = sweep ? (layout & 1 ? 512 : 256) : chunk_blocks[layout / 2];
        const int u = sweep ? (layout < 8 ? 2 : 4) : (layout & 1 ? 8 : 4);
        // private chunks: per vectors per workgroup; sweep: ntiles tiles
        const long long per = sweep ? vecs / (1024 * u) : vecs / blocks / (256 * u) * (256 * u);
        if (per == 0) continue;
        std::vector<float> t;
        for (int r = 0; r < reps + 1 && rc == 0; ++r) {
            if ((e = hipEventRecord(e0, st)) != hipSuccess) { fail(e); break; }
            if (sweep && u == 2)
                read_probe_sweep<2><<<blocks, 1024, 0, st>>>(a, per, out);
            else if (sweep)
                read_probe_sweep<4><<<blocks, 1024, 0, st>>>(a, per, out);
            else if (u == 4)
                read_probe<4><<<blocks, 256, 0, st>>>(a, per, out);
            else
                read_probe<8><<<blocks, 256, 0, st>>>(a, per, out);
            if ((e = hipGetLastError()) != hipSuccess) { fail(e); break; }
            if ((e = hipEventRecord(e1, st)) != hipSuccess) { fail(e); break; }
            if ((e = hipEventSynchronize(e1)) != hipSuccess) { fail(e); break; }
            float ms = 0.f;
            if ((e = hipEventElapsedTime(&ms, e0, e1)) != hipSuccess) { fail(e); break; }
            if (r >= 1) t.push_back(ms);
        }
        if (rc) goto done;
        std::sort(t.begin(), t.end());
        const double b = sweep ? (double)per * 1024 * u * 16 : (double)per * blocks * 16;
        best_med = std::max(best_med, (float)(b / (t[t.size() / 2] * 1e-3) / 1e9));
        best_any = std::max(best_any, (float)(b / (t[0] * 1e-3) / 1e9));
    }
    if (gbps) *gbps = best_med;
    if (best_gbps) *best_gbps = best_any;
done:
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    (void)hipStreamSynchronize(st);
    (void)hipFree(buf);
    return rc;
}

int xsymv_copy_bandwidth(size_t bytes, int reps, void* stream, float* gbps, float* best_gbps)
{
    if (bytes < ((size_t)64 << 20) || reps <= 0) return -1;
    const hipStream_t st = (hipStream_t)stream;
    const long long vecs = (long long)(bytes / 16);
    char* buf = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    int rc = 0;
    float best_med = 0.f, best_any = 0.f;
    auto fail = [&](hipError_t e) { rc = ERR_HIP + (int)e; };
    hipError_t e;
    if ((e = hipMalloc((void**)&buf, (size_t)vecs * 32)) != hipSuccess) return ERR_HIP + (int)e;
    auto* src = reinterpret_cast<xsymv::u32x4*>(buf);
    auto* dst = src + vecs;
    fill_probe<<<4096, 256, 0, st>>>(reinterpret_cast<uint32_t*>(buf), vecs * 8);
    if ((e = hipGetLastError()) != hipSuccess) { fail(e); goto done; }
    if ((e = hipEventCreate(&e0)) != hipSuccess || (e = hipEventCreate(&e1)) != hipSuccess) {
        fail(e);
        goto done;
    }
    // layouts: {2048, 8192} workgroups x {4, 8} vectors in flight per lane
    for (int layout = 0; layout < 4; ++layout) {
        const int blocks = (layout & 2) ? 8192 : 2048;
        const int u = (layout & 1) ? 8 : 4;
        const long long per = vecs / blocks / (256 * u) * (256 * u);
        if (per == 0) continue;
        std::vector<float> t;
        for (int r = 0; r < reps + 1 && rc == 0; ++r) {
            if ((e = hipEventRecord(e0, st)) != hipSuccess) { fail(e); break; }
            if (u == 4)
                copy_probe<4><<<blocks, 256, 0, st>>>(src, dst, per);
            else
                copy_probe<8><<<blocks, 256, 0, st>>>(src, dst, per);
            if ((e = hipGetLastError()) != hipSuccess) { fail(e); break; }
            if ((e = hipEventRecord(e1, st)) != hipSuccess) { fail(e); break; }
            if ((e = hipEventSynchronize(e1)) != hipSuccess) { fail(e); break; }
            float ms = 0.f;
            if ((e = hipEventElapsedTime(&ms, e0, e1)) != hipSuccess) { fail(e); break; }
            if (r >= 1) t.push_back(ms);
        }
        if (rc) goto done;
        std::sort(t.begin(), t.end());
        const double b = 2.0 * (double)per * blocks * 16;  // read + written
        best_med = std::max(best_med, (float)(b / (t[t.size() / 2] * 1e-3) / 1e9));
        best_any = std::max(best_any, (float)(b / (t[0] * 1e-3) / 1e9));
    }
    if (gbps) *gbps = best_med;
    if (best_gbps) *best_gbps = best_any;
done:
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    (void)hipStreamSynchronize(st);
    (void)hipFree(buf);
    return rc;
}

int xsymv_set_workspace(void* dev_ptr, size_t bytes, void* stream)
{
    if (!dev_ptr && bytes != 0) return -2;
    int dev = 0;
    XSYMV_HIP(hipGetDevice(&dev));
    DeviceState* ds = device_state(dev);
    std::lock_guard<std::mutex> lk(ds->mu);
    const hipStream_t st = (hipStream_t)stream;
    auto it = ds->workspaces.find(st);
    if (it != ds->workspaces.end()) {
        // the previous buffer may still be in use by work queued on this stream
        XSYMV_HIP(hipStreamSynchronize(st));
        if (it->second.owned && it->second.ptr) XSYMV_HIP(hipFree(it->second.ptr));
        ds->workspaces.erase(it);
    }
    if (dev_ptr) ds->workspaces[st] = Workspace{dev_ptr, bytes, false};
    return 0;
}

int xsymv_release(void)
{
    int dev = 0;
    XSYMV_HIP(hipGetDevice(&dev));
    DeviceState* ds = device_state(dev);
    // Lock first, so that no call can enqueue work on a buffer between the
    // synchronisation and the frees.
    std::lock_guard<std::mutex> lk(ds->mu);
    XSYMV_HIP(hipDeviceSynchronize());
    // Every entry is dropped from its map whether or not its free succeeded,
    // so a later call or release never reuses or frees it again; the first
    // error is returned after all frees were attempted.
    hipError_t first = hipSuccess;
    auto note = [&](hipError_t e) {
        if (e != hipSuccess && first == hipSuccess) first = e;
    };
    for (auto& kv : ds->workspaces)
        if (kv.second.owned && kv.second.ptr) note(hipFree(kv.second.ptr));
    ds->workspaces.clear();
    for (auto& kv : ds->plans) {
        Plan* p = kv.second.get();
        note(hipFree(p->d_tiles));
        note(hipFree(p->d_slot_base));
        note(hipHostFree(p->h_tiles));
        note(hipHostFree(p->h_slot_base));
    }
    ds->plans.clear();
    for (auto& kv : ds->strip_plans) {
        note(hipFree(kv.second->d_blocks));
        note(hipHostFree(kv.second->h_pinned));
    }
    ds->strip_plans.clear();
    for (auto& kv : ds->shard_plans) {
        note(hipFree(kv.second->d_blocks));
        note(hipHostFree(kv.second->h_pinned));
    }
    ds->shard_plans.clear();
    for (auto& kv : ds->gemv_plans) {
        note(hipFree(kv.second->d_blocks));
        note(hipHostFree(kv.second->h_pinned));
    }
    ds->gemv_plans.clear();
    return first == hipSuccess ? 0 : ERR_HIP + (int)first;
}

int xsymv_num_configs(int prec) { return num_configs(prec); }

int xsymv_config_info(int prec, int idx, int* waves, int* cols_per_wave, int* stripes,
                      int* rows_per_stripe, int* nontemporal, int* x_in_lds, int* column_runs)
{
    ConfigInfo ci;
    if (!config_info(prec, idx, &ci)) return -1;
    if (x_in_lds) *x_in_lds = ci.XLDS;
    if (column_runs) *column_runs = ci.RUNS;
    if (waves) *waves = ci.W;
    if (cols_per_wave) *cols_per_wave = ci.CW;
    if (stripes) *stripes = ci.S;
    if (rows_per_stripe) *rows_per_stripe = ci.H;
    if (nontemporal) *nontemporal = ci.NT;
    return 0;
}

int xsymv_select_config(int prec, char uplo, int n_lo, int n_hi, int idx)
{
    if (prec < 0 || prec > 4) return -1;
    bool upper;
    if (uplo == 'U' || uplo == 'u')
        upper = true;
    else if (uplo == 'L' || uplo == 'l')
        upper = false;
    else
        return -1;
    if (idx < -1 || idx >= num_configs(prec) || n_lo > n_hi) return -1;
    std::lock_guard<std::mutex> lk(g_rules_mu);
    g_rules[prec][upper ? 1 : 0].push_back(Rule{n_lo, n_hi, idx});
    return 0;
}

int xsymv_current_config(int prec, char uplo, int n)
{
    if (prec < 0 || prec > 4) return -1;
    return pick_config(prec, uplo == 'U' || uplo == 'u', n, 0);
}

int xsymv_current_config_lda(int prec, char uplo, int n, int lda)
{
    static const size_t elem[5] = {4, 8, 8, 16, 16};
    if (prec < 0 || prec > 4 || lda < 1) return -1;
    return pick_config(prec, uplo == 'U' || uplo == 'u', n, stride_class(lda, elem[prec]));
}

int xsymv_timing_enable(int on)
{
    std::lock_guard<std::mutex> tl(g_time_mu);
    if (on < 0 || on > 2) return -1;
    g_timing = on;
    return 0;
}

int xsymv_timing_read(float* main_ms, float* merge_ms, int max)
{
    std::vector<TimedCall> calls;
    {
        std::lock_guard<std::mutex> tl(g_time_mu);
        calls.swap(g_timed);
    }
    int k = 0;
    int err = 0;
    for (auto& c : calls) {
        if (!err) {
            // the last event of the call; whole-call records have no e1
            hipError_t e = hipEventSynchronize(c.e2 ? c.e2 : c.e1);
            float a = 0.f, b = 0.f;
            if (e == hipSuccess) e = hipEventElapsedTime(&a, c.e0, c.e1 ? c.e1 : c.e2);
            if (e == hipSuccess && c.e1 && c.e2) e = hipEventElapsedTime(&b, c.e1, c.e2);
            if (e != hipSuccess) {
                err = ERR_HIP + (int)e;
            } else if (k < max) {
                if (main_ms) main_ms[k] = a;
                if (merge_ms) merge_ms[k] = b;
                ++k;
            }
        }
        (void)hipEventDestroy(c.e0);
        if (c.e1) (void)hipEventDestroy(c.e1);
        if (c.e2) (void)hipEventDestroy(c.e2);
    }
    return err ? err : k;
}

int xsymv_autotune(int prec, char uplo, int n, int n_lo, int n_hi, int reps, void* stream,
                   int* best_idx, float* ms, int max_cfg)
{
    return xsymv_autotune_lda(prec, uplo, n, n, n_lo, n_hi, reps, stream, best_idx, ms, max_cfg);
}

int xsymv_autotune_lda(int prec, char uplo, int n, int lda, int n_lo, int n_hi, int reps,
                       void* stream, int* best_idx, float* ms, int max_cfg)
{
    if (prec < 0 || prec > 4 || n_lo > n_hi || n <= 0 || reps <= 0 || lda < n) return -1;
    if (!(uplo == 'U' || uplo == 'u' || uplo == 'L' || uplo == 'l')) return -1;
    int best = 0;
    hipStream_t st = (hipStream_t)stream;
    int rc;
    switch (prec) {
    case XSYMV_S: rc = autotune_for<float>(uplo, n, lda, reps, st, &best, ms, max_cfg); break;
    case XSYMV_D: rc = autotune_for<double>(uplo, n, lda, reps, st, &best, ms, max_cfg); break;
    case XSYMV_C: rc = autotune_for<cf32>(uplo, n, lda, reps, st, &best, ms, max_cfg); break;
    case XSYMV_Z: rc = autotune_for<cf64>(uplo, n, lda, reps, st, &best, ms, max_cfg); break;
    default: rc = autotune_for<ddreal>(uplo, n, lda, reps, st, &best, ms, max_cfg); break;
    }
    if (rc) return rc;
    if (best_idx) *best_idx = best;
    return xsymv_select_config(prec, uplo, n_lo, n_hi, best);
}

int xsymv_save_config(const char* path)
{
    if (!path) return -1;
    FILE* f = std::fopen(path, "w");
    if (!f) return -1;
    std::fprintf(f, "{\"library\": \"%s\", \"rules\": [", xsymv_version());
    bool first = true;
    {
        std::lock_guard<std::mutex> lk(g_rules_mu);
        for (int p = 0; p < 5; ++p)
            for (int u = 0; u < 2; ++u)
                for (const Rule& r : g_rules[p][u]) {
                    ConfigInfo ci;
                    if (r.idx < 0 || !config_info(p, r.idx, &ci)) continue;
                    std::fprintf(f,
                                 "%s\n  {\"prec\": \"%c\", \"uplo\": \"%c\", \"n_lo\": %d, "
                                 "\"n_hi\": %d, \"waves\": %d, \"cols_per_wave\": %d, "
                                 "\"stripes\": %d, \"nontemporal\": %d, \"x_in_lds\": %d, "
                                 "\"column_runs\": %d}",
                                 first ? "" : ",", PREC_CHARS[p], u ? 'U' : 'L', r.n_lo, r.n_hi,
                                 ci.W, ci.CW, ci.S, ci.NT, ci.XLDS, ci.RUNS);
                    first = false;
                }
    }
    std::fprintf(f, "\n]}\n");
    return std::fclose(f) == 0 ? 0 : -1;
}

int xsymv_load_config(const char* path)
{
    if (!path) return -1;
    FILE* f = std::fopen(path, "r");
    if (!f) return -1;
    std::string text;
    char buf[4096];
    size_t k;
    while ((k = std::fread(buf, 1, sizeof buf, f)) > 0) text.append(buf, k);
    std::fclose(f);
    std::vector<JsonRule> rules;
    if (!parse_rules(text, rules)) return -2;
    int loaded = 0;
    for (const JsonRule& r : rules) {
        auto get = [&](const char* key) -> const std::string* {
            auto it = r.kv.find(key);
            return it == r.kv.end() ? nullptr : &it->second;
        };
        const std::string *ps = get("prec"), *us = get("uplo");
        const char* keys[8] = {"n_lo", "n_hi", "waves", "cols_per_wave", "stripes", "nontemporal",
                               "x_in_lds", "column_runs"};
        int v[8];
        bool ok = ps && us && ps->size() == 1 && us->size() == 1;
        for (int i = 0; i < 8 && ok; ++i) {
            const std::string* s = get(keys[i]);
            ok = s != nullptr;
            if (ok) v[i] = std::atoi(s->c_str());
        }
        if (!ok) continue;
        const int prec = prec_of_char((*ps)[0]);
        if (prec < 0) continue;
        const int idx = find_config(prec, v[2], v[3], v[4], v[5], v[6], v[7]);
        if (idx < 0) continue;
        if (xsymv_select_config(prec, (*us)[0], v[0], v[1], idx) == 0) ++loaded;
    }
    return loaded;
}

int xsymv_clear_config(void)
{
    std::lock_guard<std::mutex> lk(g_rules_mu);
    for (int p = 0; p < 5; ++p)
        for (int u = 0; u < 2; ++u) g_rules[p][u].clear();
    return 0;
}

int xsymv_config_workgroups(int prec, int idx, char uplo)
{
    const bool upper = (uplo == 'U' || uplo == 'u');
    const void* k = nullptr;
    int threads = 0;
    switch (prec) {
#define XSYMV_K(T)                                                                       \
    {                                                                                    \
        if (idx < 0 || idx >= (int)kernel_sets<T>().size()) return -1;                   \
        const auto& ks = kernel_sets<T>()[idx];                                          \
        if (!ks.info.strip()) return 0;                                                  \
        k = (const void*)(upper ? ks.strip_upper : ks.strip_lower);                      \
        threads = 64 * ks.info.W;                                                        \
        break;                                                                           \
    }
    case XSYMV_S: XSYMV_K(float)
    case XSYMV_D: XSYMV_K(double)
    case XSYMV_C: XSYMV_K(cf32)
    case XSYMV_Z: XSYMV_K(cf64)
    case XSYMV_W: XSYMV_K(ddreal)
#undef XSYMV_K
    default: return -1;
    }
    int G = 0;
    const int rc = resident_blocks(k, threads, &G);
    return rc ? -rc : G;
}

int xsymv_strip_plan(char uplo, int n, int R, int G, int split, int* blocks4, int max_blocks,
                     int* strip_base, int* seg_base, int max_strips)
{
    if (!(uplo == 'U' || uplo == 'u' || uplo == 'L' || uplo == 'l') || n <= 0 || R <= 0 ||
        G <= 0 || split < 0 || split > 2)
        return -1;
    std::vector<StripBlock> blocks;
    std::vector<int> sb, segb;
    int NS = 0;
    build_strip_plan_host(uplo == 'U' || uplo == 'u', n, R, G, split, blocks, sb, segb, NS);
    if ((int)blocks.size() > max_blocks || NS + 1 > max_strips) return -2;
    for (size_t b = 0; b < blocks.size(); ++b) {
        blocks4[4 * b + 0] = blocks[b].u0;
        blocks4[4 * b + 1] = blocks[b].u1;
        blocks4[4 * b + 2] = blocks[b].slot0;
        blocks4[4 * b + 3] = blocks[b].strip0;
    }
    std::copy(sb.begin(), sb.end(), strip_base);
    std::copy(segb.begin(), segb.end(), seg_base);
    return (int)blocks.size();
}

int xsymv_shard_plan(char uplo, int n, int R, int G, int split, int panel, int nshards, int shard,
                     int* blocks4, int max_blocks, int* strip_base, int* seg_base, int* col0,
                     int max_strips)
{
    if (!(uplo == 'U' || uplo == 'u' || uplo == 'L' || uplo == 'l') || n <= 0 || R <= 0 ||
        G <= 0 || split < 0 || split > 2 || panel <= 0 || nshards <= 0 || shard < 0 ||
        shard >= nshards)
        return -1;
    std::vector<int> cols, c0;
    shard_columns_host(n, panel, nshards, shard, cols);
    if (cols.empty()) return 0;
    std::vector<StripBlock> blocks;
    std::vector<int> sb, segb;
    int NS = 0;
    build_strip_plan_host(uplo == 'U' || uplo == 'u', n, R, G, split, blocks, sb, segb, NS, &cols,
                          &c0);
    if ((int)blocks.size() > max_blocks || NS + 1 > max_strips) return -2;
    for (size_t b = 0; b < blocks.size(); ++b) {
        blocks4[4 * b + 0] = blocks[b].u0;
        blocks4[4 * b + 1] = blocks[b].u1;
        blocks4[4 * b + 2] = blocks[b].slot0;
        blocks4[4 * b + 3] = blocks[b].strip0;
    }
    std::copy(sb.begin(), sb.end(), strip_base);
    std::copy(segb.begin(), segb.end(), seg_base);
    std::copy(c0.begin(), c0.end(), col0);
    return (int)blocks.size();
}

int xgemv_num_configs(int prec)
{
    switch (prec) {
    case XSYMV_S: return (int)gemv_kernel_sets<float>().size();
    case XSYMV_D: return (int)gemv_kernel_sets<double>().size();
    case XSYMV_C: return (int)gemv_kernel_sets<cf32>().size();
    case XSYMV_Z: return (int)gemv_kernel_sets<cf64>().size();
    case XSYMV_W: return (int)gemv_kernel_sets<ddreal>().size();
    default: return -1;
    }
}

int xgemv_config_info(int prec, int idx, int* waves, int* stripes_per_wave, int* cols_per_group,
                      int* nontemporal, int* rows_per_strip)
{
    if (idx < 0 || idx >= xgemv_num_configs(prec)) return -1;
    int W = 0, SW = 0, G = 0, NT = 0, R = 0;
    switch (prec) {
#define XSYMV_K(T)                                                                       \
    {                                                                                    \
        const auto& k = gemv_kernel_sets<T>()[idx];                                      \
        W = k.W; SW = k.SW; G = k.G; NT = k.NT; R = k.R();                               \
        break;                                                                           \
    }
    case XSYMV_S: XSYMV_K(float)
    case XSYMV_D: XSYMV_K(double)
    case XSYMV_C: XSYMV_K(cf32)
    case XSYMV_Z: XSYMV_K(cf64)
    default: XSYMV_K(ddreal)
#undef XSYMV_K
    }
    if (waves) *waves = W;
    if (stripes_per_wave) *stripes_per_wave = SW;
    if (cols_per_group) *cols_per_group = G;
    if (nontemporal) *nontemporal = NT;
    if (rows_per_strip) *rows_per_strip = R;
    return 0;
}

int xgemv_select_config(int prec, int idx)
{
    if (prec < 0 || prec > 4 || idx < -1 || idx >= xgemv_num_configs(prec)) return -1;
    g_gemv_idx[prec].store(idx);
    return 0;
}

int xgemv_current_config(int prec, char trans, int m, int n)
{
    int tr = 0;
    // the argument checks of a call (transposition only; no data)
    if (check_gemv_args(trans, 0, 0, nullptr, 1, nullptr, 1, nullptr, 1, &tr)) return -1;
    if (m < 0 || n < 0) return -1;
    switch (prec) {
    case XSYMV_S: return gemv_pick<float>(tr, m, n);
    case XSYMV_D: return gemv_pick<double>(tr, m, n);
    case XSYMV_C: return gemv_pick<cf32>(tr, m, n);
    case XSYMV_Z: return gemv_pick<cf64>(tr, m, n);
    case XSYMV_W: return gemv_pick<ddreal>(tr, m, n);
    default: return -1;
    }
}

size_t xgemv_workspace_bytes(int prec, char trans, int m, int n)
{
    switch (prec) {
    case XSYMV_S: return gemv_ws_bytes<float>(trans, m, n);
    case XSYMV_D: return gemv_ws_bytes<double>(trans, m, n);
    case XSYMV_C: return gemv_ws_bytes<cf32>(trans, m, n);
    case XSYMV_Z: return gemv_ws_bytes<cf64>(trans, m, n);
    case XSYMV_W: return gemv_ws_bytes<ddreal>(trans, m, n);
    default: return (size_t)-1;
    }
}

int xgemv_plan(int m, int n, int R, int G, int* blocks4, int max_blocks, int* seg_base,
               int max_strips)
{
    if (m <= 0 || n <= 0 || R <= 0 || G <= 0) return -1;
    std::vector<StripBlock> blocks;
    std::vector<int> segb;
    int NS = 0;
    build_gemv_plan_host(m, n, R, G, blocks, segb, NS);
    if ((int)blocks.size() > max_blocks || NS + 1 > max_strips) return -2;
    for (size_t b = 0; b < blocks.size(); ++b) {
        blocks4[4 * b + 0] = blocks[b].u0;
        blocks4[4 * b + 1] = blocks[b].u1;
        blocks4[4 * b + 2] = blocks[b].slot0;
        blocks4[4 * b + 3] = blocks[b].strip0;
    }
    std::copy(segb.begin(), segb.end(), seg_base);
    return (int)blocks.size();
}

int xsyr2_num_configs(int prec)
{
    switch (prec) {
    case XSYMV_S: return (int)syr2_kernel_sets<float>().size();
    case XSYMV_D: return (int)syr2_kernel_sets<double>().size();
    case XSYMV_C: return (int)syr2_kernel_sets<cf32>().size();
    case XSYMV_Z: return (int)syr2_kernel_sets<cf64>().size();
    case XSYMV_W: return (int)syr2_kernel_sets<ddreal>().size();
    default: return -1;
    }
}

int xsyr2_config_info(int prec, int idx, int* waves, int* stripes_per_wave, int* cols_per_group,
                      int* nontemporal, int* split, int* rows_per_strip)
{
    if (idx < 0 || idx >= xsyr2_num_configs(prec)) return -1;
    int W = 0, SW = 0, G = 0, NT = 0, SP = 0, R = 0;
    switch (prec) {
#define XSYMV_K(T)                                                                       \
    {                                                                                    \
        const auto& k = syr2_kernel_sets<T>()[idx];                                      \
        W = k.W; SW = k.SW; G = k.G; NT = k.NT; SP = k.split; R = k.R();                 \
        break;                                                                           \
    }
    case XSYMV_S: XSYMV_K(float)
    case XSYMV_D: XSYMV_K(double)
    case XSYMV_C: XSYMV_K(cf32)
    case XSYMV_Z: XSYMV_K(cf64)
    default: XSYMV_K(ddreal)
#undef XSYMV_K
    }
    if (waves) *waves = W;
    if (stripes_per_wave) *stripes_per_wave = SW;
    if (cols_per_group) *cols_per_group = G;
    if (nontemporal) *nontemporal = NT;
    if (split) *split = SP;
    if (rows_per_strip) *rows_per_strip = R;
    return 0;
}

int xsyr2_select_config(int prec, int idx)
{
    if (prec < 0 || prec > 4 || idx < -1 || idx >= xsyr2_num_configs(prec)) return -1;
    g_syr2_idx[prec].store(idx);
    return 0;
}

int xsyr2_current_config(int prec, char uplo, int n)
{
    bool upper = false;
    if (uplo == 'U' || uplo == 'u')
        upper = true;
    else if (uplo != 'L' && uplo != 'l')
        return -1;
    if (n < 0) return -1;
    switch (prec) {
    case XSYMV_S: return syr2_pick<float>(upper, n);
    case XSYMV_D: return syr2_pick<double>(upper, n);
    case XSYMV_C: return syr2_pick<cf32>(upper, n);
    case XSYMV_Z: return syr2_pick<cf64>(upper, n);
    case XSYMV_W: return syr2_pick<ddreal>(upper, n);
    default: return -1;
    }
}

int xtrmv_num_configs(int prec)
{
    switch (prec) {
    case XSYMV_S: return (int)trmv_kernel_sets<float>().size();
    case XSYMV_D: return (int)trmv_kernel_sets<double>().size();
    case XSYMV_C: return (int)trmv_kernel_sets<cf32>().size();
    case XSYMV_Z: return (int)trmv_kernel_sets<cf64>().size();
    case XSYMV_W: return (int)trmv_kernel_sets<ddreal>().size();
    default: return -1;
    }
}

int xtrmv_config_info(int prec, int idx, int* waves, int* stripes_per_wave, int* cols_per_group,
                      int* nontemporal, int* split, int* rows_per_strip)
{
    if (idx < 0 || idx >= xtrmv_num_configs(prec)) return -1;
    int W = 0, SW = 0, G = 0, NT = 0, SP = 0, R = 0;
    switch (prec) {
#define XSYMV_K(T)                                                                       \
    {                                                                                    \
        const auto& k = trmv_kernel_sets<T>()[idx];                                      \
        W = k.W; SW = k.SW; G = k.G; NT = k.NT; SP = k.split; R = k.R();                 \
        break;                                                                           \
    }
    case XSYMV_S: XSYMV_K(float)
    case XSYMV_D: XSYMV_K(double)
    case XSYMV_C: XSYMV_K(cf32)
    case XSYMV_Z: XSYMV_K(cf64)
    default: XSYMV_K(ddreal)
#undef XSYMV_K
    }
    if (waves) *waves = W;
    if (stripes_per_wave) *stripes_per_wave = SW;
    if (cols_per_group) *cols_per_group = G;
    if (nontemporal) *nontemporal = NT;
    if (split) *split = SP;
    if (rows_per_strip) *rows_per_strip = R;
    return 0;
}

int xtrmv_select_config(int prec, int idx)
{
    if (prec < 0 || prec > 4 || idx < -1 || idx >= xtrmv_num_configs(prec)) return -1;
    g_trmv_idx[prec].store(idx);
    return 0;
}

int xtrmv_current_config(int prec, char uplo, char trans, int n)
{
    bool upper = false, unit = false;
    int tr = 0;
    // the argument checks of a call with n = 0
    if (check_trmv_args(uplo, trans, 'N', 0, nullptr, 1, nullptr, 1, &upper, &tr, &unit))
        return -1;
    if (n < 0) return -1;
    switch (prec) {
    case XSYMV_S: return trmv_pick<float>(upper, tr, n);
    case XSYMV_D: return trmv_pick<double>(upper, tr, n);
    case XSYMV_C: return trmv_pick<cf32>(upper, tr, n);
    case XSYMV_Z: return trmv_pick<cf64>(upper, tr, n);
    case XSYMV_W: return trmv_pick<ddreal>(upper, tr, n);
    default: return -1;
    }
}

size_t xtrmv_workspace_bytes(int prec, char uplo, char trans, int n)
{
    switch (prec) {
    case XSYMV_S: return trmv_ws_bytes<float>(uplo, trans, n);
    case XSYMV_D: return trmv_ws_bytes<double>(uplo, trans, n);
    case XSYMV_C: return trmv_ws_bytes<cf32>(uplo, trans, n);
    case XSYMV_Z: return trmv_ws_bytes<cf64>(uplo, trans, n);
    case XSYMV_W: return trmv_ws_bytes<ddreal>(uplo, trans, n);
    default: return (size_t)-1;
    }
}

int xsymv_shard_columns(int n, int panel, int nshards, int shard, int* cols)
{
    if (n < 0 || panel <= 0 || nshards <= 0 || shard < 0 || shard >= nshards) return -1;
    std::vector<int> c;
    shard_columns_host(n, panel, nshards, shard, c);
    if (cols) std::copy(c.begin(), c.end(), cols);
    return (int)c.size();
}

size_t xsymv_shard_workspace_bytes(int prec, char uplo, int n, int panel, int nshards, int shard)
{
    switch (prec) {
    case XSYMV_S: return shard_ws_bytes<float>(uplo, n, panel, nshards, shard);
    case XSYMV_D: return shard_ws_bytes<double>(uplo, n, panel, nshards, shard);
    case XSYMV_C: return shard_ws_bytes<cf32>(uplo, n, panel, nshards, shard);
    case XSYMV_Z: return shard_ws_bytes<cf64>(uplo, n, panel, nshards, shard);
    case XSYMV_W: return shard_ws_bytes<ddreal>(uplo, n, panel, nshards, shard);
    default: return (size_t)-1;
    }
}

const char* xsymv_version(void) { return "xsymv-gfx950 0.1"; }

}  // extern "C"
