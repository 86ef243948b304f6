// C-ABI of libgat.so (declared in include/gat.h): host-side argument checks, plan
// layout, and dispatch to the gfx950 kernels.  Every check runs before anything is
// enqueued; no exception leaves this file.
#include "gat.h"

#include <limits.h>
#include <string.h>

#include <atomic>

#include "kernels.hpp"
#include "linear.hpp"

namespace gat {
hipError_t launch_spmm_agg(int, int, int, const int32_t*, const int32_t*, int64_t, int64_t, const float*,
                           const void*, const void*, const void*, float, float*, const PlanView*, hipStream_t);
hipError_t launch_spmm_softagg(int, int, int, const int32_t*, const int32_t*, int64_t, int64_t, const float*,
                               const void*, const void*, const void*, float, float*, const PlanView*, hipStream_t);
hipError_t launch_spmm_layer(int, int, int, const int32_t*, const int32_t*, int64_t, int64_t, const float*,
                             const void*, const void*, const void*, float, float*, const PlanView*, hipStream_t);

hipError_t launch_spmm(int mode, int dtype, int H, int D, const int32_t* row_ptr, const int32_t* col_idx,
                       int64_t n_rows, int64_t n_src, const float* scores, const void* q, const void* k, const void* v, float scale,
                       float* out, const PlanView* plan, hipStream_t stream) {
    switch (mode) {
        case kAgg:
            return launch_spmm_agg(dtype, H, D, row_ptr, col_idx, n_rows, n_src, scores, q, k, v, scale, out, plan, stream);
        case kSoftAgg:
            return launch_spmm_softagg(dtype, H, D, row_ptr, col_idx, n_rows, n_src, scores, q, k, v, scale, out, plan,
                                       stream);
        case kLayer:
            return launch_spmm_layer(dtype, H, D, row_ptr, col_idx, n_rows, n_src, scores, q, k, v, scale, out, plan,
                                     stream);
        default:
            return hipErrorInvalidValue;
    }
}
}  // namespace gat

namespace {

constexpr uint32_t kPlanMagic = 0x47415450u;   // "GATP"
constexpr int64_t kMaxIndex = INT32_MAX;
// Edge positions advance in chunks of up to 64 inside int32 loop counters; keep headroom.
constexpr int64_t kMaxEdges = INT32_MAX - 4096;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool size_ok(int64_t n) { return n >= 0 && n <= kMaxIndex; }

bool edges_ok(int64_t n) { return n >= 0 && n <= kMaxEdges; }

bool dtype_ok(gat_dtype dt) { return dt == GAT_F32 || dt == GAT_BF16; }

bool heads_ok(int heads) { return heads == 1 || heads == 2 || heads == 4 || heads == 8 || heads == 16; }

bool shape_ok(int heads, int head_dim) {
    return heads_ok(heads) && (head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128) &&
           heads * head_dim <= 1024;
}

struct Layout {
    int64_t n_blocks, seg_cap, hub_cap, hubseg_cap, state_floats;
    size_t off_counts, off_blocks, off_segs, off_hubs, off_partials, total;
};

// Table capacities.  Segments: at most E/seg_len + (number of non-short rows), and a
// non-short row has deg > short_max, so there are at most E/(short_max+1) of them.
// Hubs have deg > seg_len: at most E/(seg_len+1).  A hub row of degree d has
// ceil(d/seg_len) < 2d/seg_len segments, so hub segments number at most 2E/seg_len.
Layout plan_layout(int64_t n_rows, int64_t n_edges, int heads, int head_dim, int short_max, int seg_len) {
    Layout L{};
    L.n_blocks = (n_rows + gat::kPlanRowsPerBlock - 1) / gat::kPlanRowsPerBlock;
    int64_t nonshort = n_edges / ((int64_t)short_max + 1);
    if (nonshort > n_rows) nonshort = n_rows;
    L.seg_cap = n_edges / seg_len + nonshort + 1;
    L.hub_cap = n_edges / ((int64_t)seg_len + 1);
    if (L.hub_cap > n_rows) L.hub_cap = n_rows;
    L.hub_cap += 1;
    L.hubseg_cap = 2 * (n_edges / seg_len) + 2;
    if (L.hubseg_cap > L.seg_cap) L.hubseg_cap = L.seg_cap;
    L.state_floats = (int64_t)heads * (head_dim + 2);
    size_t off = 0;
    L.off_counts = off;
    off = align_up(off + 8 * sizeof(int32_t));
    L.off_blocks = off;
    off = align_up(off + (size_t)(L.n_blocks + 1) * 16);
    L.off_segs = off;
    off = align_up(off + (size_t)L.seg_cap * 16);
    L.off_hubs = off;
    off = align_up(off + (size_t)L.hub_cap * 16);
    L.off_partials = off;
    off = align_up(off + (size_t)L.hubseg_cap * (size_t)L.state_floats * sizeof(float));
    L.total = off;
    return L;
}

void resolve_thresholds(int& short_max, int& seg_len) {
    if (short_max < 0) short_max = GAT_DEFAULT_SHORT_MAX;
    if (seg_len <= 0) seg_len = GAT_DEFAULT_SEG_LEN;
}

gat::PlanView plan_view(const gat_plan* p) {
    gat::PlanView v{};
    char* base = static_cast<char*>(p->ws);
    v.counts = reinterpret_cast<const int32_t*>(base + p->off_counts);
    v.segs = reinterpret_cast<const int4*>(base + p->off_segs);
    v.hubs = reinterpret_cast<const int4*>(base + p->off_hubs);
    v.partials = reinterpret_cast<float*>(base + p->off_partials);
    v.state_floats = p->state_floats;
    v.seg_capacity = p->seg_capacity;
    v.hub_capacity = p->hub_capacity;
    v.hubseg_capacity = p->hubseg_capacity;
    v.short_max = p->short_max;
    v.seg_len = p->seg_len;
    return v;
}

// A plan usable for a call on this row_ptr array and (n_rows, n_edges), needing `floats` floats of
// state per hub segment.  A plan built from another array (even one of the same sizes) would
// leave the rows it does not cover unwritten, so it is refused.
gat_status check_plan(const gat_plan* p, const int32_t* row_ptr, int64_t n_rows, int64_t n_edges, int64_t floats) {
    if (p->magic != kPlanMagic || p->ws == nullptr) return GAT_ERR_ARGS;
    if (p->row_ptr != row_ptr) return GAT_ERR_WORKSPACE;
    if (p->n_rows != n_rows || p->n_edges != n_edges) return GAT_ERR_WORKSPACE;
    if (floats > p->state_floats) return GAT_ERR_WORKSPACE;
    return GAT_OK;
}

gat_status hip_status(hipError_t e) { return e == hipSuccess ? GAT_OK : GAT_ERR_HIP; }

// Fills *p for a plan of layout L in ws and enqueues its build on row_ptr.
hipError_t build_plan(const int32_t* row_ptr, int64_t n_rows, int64_t n_edges, int heads, int head_dim,
                      int short_max, int seg_len, const Layout& L, void* ws, size_t ws_bytes, gat_plan* p,
                      hipStream_t stream) {
    memset(p, 0, sizeof *p);
    p->n_rows = n_rows;
    p->n_edges = n_edges;
    p->short_max = short_max;
    p->seg_len = seg_len;
    p->heads = heads;
    p->head_dim = head_dim;
    p->state_floats = L.state_floats;
    p->seg_capacity = L.seg_cap;
    p->hub_capacity = L.hub_cap;
    p->hubseg_capacity = L.hubseg_cap;
    p->n_blocks = L.n_blocks;
    p->ws = ws;
    p->ws_bytes = ws_bytes;
    p->row_ptr = row_ptr;
    p->off_counts = L.off_counts;
    p->off_blocks = L.off_blocks;
    p->off_segs = L.off_segs;
    p->off_hubs = L.off_hubs;
    p->off_partials = L.off_partials;
    p->magic = kPlanMagic;
    char* base = static_cast<char*>(ws);
    return gat::launch_plan(row_ptr, n_rows, short_max, seg_len, reinterpret_cast<int4*>(base + L.off_blocks),
                            L.n_blocks, reinterpret_cast<int32_t*>(base + L.off_counts),
                            reinterpret_cast<int4*>(base + L.off_segs), reinterpret_cast<int4*>(base + L.off_hubs),
                            gat::PlanCaps{L.seg_cap, L.hub_cap, L.hubseg_cap}, stream);
}

// ------------------------------------------------------------------------------ transposed view
constexpr uint32_t kCscMagic = 0x47415443u;   // "GATC"

struct CscLayout {
    gat::RadixPlan sort;
    size_t off_col_ptr, off_row_idx, off_rows, off_keys[2], off_vals[2], off_rows2, off_hist, off_sums, off_stage,
        off_plan;
    Layout plan;
    size_t total;
};

CscLayout csc_layout(int64_t n_rows, int64_t n_src, int64_t n_edges, int heads, int head_dim) {
    (void)n_rows;
    CscLayout C{};
    C.sort = gat::radix_plan(n_src);   // columns are < n_src
    const int64_t hist = (int64_t)gat::kRadixMaxBins * gat::radix_tiles(n_edges);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    C.off_col_ptr = take((size_t)(n_src + 1) * 4);
    C.off_row_idx = take((size_t)n_edges * 4);
    C.off_rows = take((size_t)n_edges * 4);
    for (int b = 0; b < 2; ++b) {
        C.off_keys[b] = take((size_t)n_edges * 4);
        C.off_vals[b] = take((size_t)n_edges * 4);
    }
    C.off_rows2 = take((size_t)n_edges * 4);   // the rows between passes (row_idx takes the last pass)
    C.off_hist = take((size_t)hist * 4);
    C.off_sums = take((size_t)(gat::scan_tiles(hist) + 1) * 4);
    C.off_stage = take((size_t)n_edges * heads * 4);
    C.plan = plan_layout(n_src, n_edges, heads, head_dim, GAT_DEFAULT_SHORT_MAX, GAT_DEFAULT_SEG_LEN);
    C.off_plan = take(C.plan.total);
    C.total = off;
    return C;
}

// A gat_csc usable for a call on this graph with this shape.
gat_status check_csc(const gat_csc* c, int64_t n_rows, int64_t n_src, int64_t n_edges, int heads, int head_dim) {
    if (c->magic != kCscMagic || c->ws == nullptr) return GAT_ERR_ARGS;
    if (c->n_rows != n_rows || c->n_src != n_src || c->n_edges != n_edges) return GAT_ERR_WORKSPACE;
    if (c->heads != heads || c->head_dim != head_dim) return GAT_ERR_WORKSPACE;
    return GAT_OK;
}

template <typename T>
T* at(const gat_csc* c, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(c->ws) + off);
}

// Layer-backward workspace: scores, alpha and the edge gradient, each [E,H] fp32.
struct BwdLayout {
    size_t off_scores, off_alpha, off_grad, total;
};

BwdLayout bwd_layout(int64_t n_edges, int heads) {
    BwdLayout B{};
    size_t off = 0;
    B.off_scores = off;
    off = align_up(off + (size_t)n_edges * heads * 4);
    B.off_alpha = off;
    off = align_up(off + (size_t)n_edges * heads * 4);
    B.off_grad = off;
    off = align_up(off + (size_t)n_edges * heads * 4);
    B.total = off > kAlign ? off : kAlign;   // never 0: 0 reports unsupported sizes
    return B;
}

// COO SDDMM backward workspace.  The two gradients are sums over the edges grouped by one
// endpoint; each side in turn sorts the edges by that endpoint (stable radix passes), builds
// the CSR of the grouping and its plan, and runs the aggregation.  Both sides reuse the same
// buffers, sized for the larger side.
struct CooBwdLayout {
    size_t off_row_ptr, off_col, off_col2, off_keys[2], off_vals[2], off_hist, off_sums, off_w, off_plan, total;
    size_t plan_bytes;
};

CooBwdLayout coo_bwd_layout(int64_t n_edges, int64_t n_src, int64_t n_dst, int heads, int head_dim) {
    CooBwdLayout C{};
    const int64_t n_max = n_src > n_dst ? n_src : n_dst;
    const int64_t hist = (int64_t)gat::kRadixMaxBins * gat::radix_tiles(n_edges);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    C.off_row_ptr = take((size_t)(n_max + 1) * 4);
    C.off_col = take((size_t)n_edges * 4);
    C.off_col2 = take((size_t)n_edges * 4);   // the other endpoint between passes (col takes the last)
    for (int b = 0; b < 2; ++b) {
        C.off_keys[b] = take((size_t)n_edges * 4);
        C.off_vals[b] = take((size_t)n_edges * 4);
    }
    C.off_hist = take((size_t)hist * 4);
    C.off_sums = take((size_t)(gat::scan_tiles(hist) + 1) * 4);
    C.off_w = take((size_t)n_edges * heads * 4);
    const size_t ps = plan_layout(n_src, n_edges, heads, head_dim, GAT_DEFAULT_SHORT_MAX, GAT_DEFAULT_SEG_LEN).total;
    const size_t pd = plan_layout(n_dst, n_edges, heads, head_dim, GAT_DEFAULT_SHORT_MAX, GAT_DEFAULT_SEG_LEN).total;
    C.plan_bytes = ps > pd ? ps : pd;
    C.off_plan = take(C.plan_bytes);
    C.total = off;
    return C;
}

std::atomic<int64_t> g_edge_grid_cap{gat::kEdgeGridDefault};

}  // namespace

int64_t gat::edge_grid_cap() { return g_edge_grid_cap.load(std::memory_order_relaxed); }

extern "C" {

int64_t gat_testing_edge_grid_cap(int64_t cap) {
    if (cap <= 0 || cap > gat::kEdgeGridDefault) cap = gat::kEdgeGridDefault;
    return g_edge_grid_cap.exchange(cap);
}


const char* gat_status_str(gat_status s) {
    switch (s) {
        case GAT_OK: return "ok";
        case GAT_ERR_NULL: return "required pointer is NULL";
        case GAT_ERR_SIZE: return "size negative or above INT32_MAX";
        case GAT_ERR_UNSUPPORTED: return "unsupported heads/head_dim/dtype";
        case GAT_ERR_WORKSPACE: return "plan workspace too small or built for other sizes";
        case GAT_ERR_ARGS: return "inconsistent arguments";
        case GAT_ERR_HIP: return "HIP launch or runtime error";
        case GAT_ERR_SCRATCH: return "graph too large for the library's fixed scratch array (GAT_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int gat_shape_supported(int heads, int head_dim) { return shape_ok(heads, head_dim) ? 1 : 0; }

size_t gat_plan_sizeof(void) { return sizeof(gat_plan); }

size_t gat_plan_workspace_bytes(int64_t n_rows, int64_t n_edges, int heads, int head_dim, int short_max,
                                int seg_len) {
    if (!size_ok(n_rows) || !edges_ok(n_edges) || !shape_ok(heads, head_dim)) return 0;
    resolve_thresholds(short_max, seg_len);
    return plan_layout(n_rows, n_edges, heads, head_dim, short_max, seg_len).total;
}

gat_status gat_plan_build(const int32_t* row_ptr, int64_t n_rows, int64_t n_edges, int heads, int head_dim,
                          int short_max, int seg_len, void* ws, size_t ws_bytes, gat_plan* plan,
                          hipStream_t stream) {
    if (plan == nullptr || row_ptr == nullptr || ws == nullptr) return GAT_ERR_NULL;
    if (!size_ok(n_rows) || !edges_ok(n_edges)) return GAT_ERR_SIZE;
    if (!shape_ok(heads, head_dim)) return GAT_ERR_UNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return GAT_ERR_ARGS;
    resolve_thresholds(short_max, seg_len);
    const Layout L = plan_layout(n_rows, n_edges, heads, head_dim, short_max, seg_len);
    if (ws_bytes < L.total) return GAT_ERR_WORKSPACE;
    gat_plan p;
    const hipError_t e = build_plan(row_ptr, n_rows, n_edges, heads, head_dim, short_max, seg_len, L, ws, ws_bytes,
                                    &p, stream);
    if (e != hipSuccess) return GAT_ERR_HIP;
    *plan = p;
    return GAT_OK;
}

gat_status gat_sddmm(const int32_t* src_idx, const int32_t* dst_idx, int64_t n_edges, const void* src_feat,
                     int64_t n_src, const void* dst_feat, int64_t n_dst, gat_dtype dtype, int heads, int head_dim,
                     float scale, float* out, hipStream_t stream) {
    if (!edges_ok(n_edges) || !size_ok(n_src) || !size_ok(n_dst)) return GAT_ERR_SIZE;
    if (!shape_ok(heads, head_dim) || !dtype_ok(dtype)) return GAT_ERR_UNSUPPORTED;
    if (n_edges == 0) return GAT_OK;
    if (!src_idx || !dst_idx || !src_feat || !dst_feat || !out) return GAT_ERR_NULL;
    if (n_src == 0 || n_dst == 0) return GAT_ERR_ARGS;   // an edge needs a source and a destination row
    return hip_status(gat::launch_sddmm(dtype, heads, head_dim, src_idx, dst_idx, n_edges, src_feat, n_src,
                                        dst_feat, n_dst, scale, out, stream));
}

gat_status gat_edge_softmax(const int32_t* row_ptr, int64_t n_rows, int64_t n_edges, int heads,
                            const float* scores, float* out, const gat_plan* plan, hipStream_t stream) {
    if (!size_ok(n_rows) || !edges_ok(n_edges)) return GAT_ERR_SIZE;
    if (!heads_ok(heads)) return GAT_ERR_UNSUPPORTED;
    if (n_rows == 0 || n_edges == 0) return GAT_OK;
    if (!row_ptr || !scores || !out) return GAT_ERR_NULL;
    gat::PlanView pv;
    if (plan) {
        const gat_status st = check_plan(plan, row_ptr, n_rows, n_edges, 2 * (int64_t)heads);
        if (st != GAT_OK) return st;
        pv = plan_view(plan);
    }
    return hip_status(gat::launch_softmax(heads, row_ptr, n_rows, scores, out, plan ? &pv : nullptr, stream));
}

gat_status gat_aggregate(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t n_src,
                         int64_t n_edges, const float* weights, const void* feat, gat_dtype dtype, int heads,
                         int head_dim, float* out, const gat_plan* plan, hipStream_t stream) {
    if (!size_ok(n_rows) || !size_ok(n_src) || !edges_ok(n_edges)) return GAT_ERR_SIZE;
    if (!shape_ok(heads, head_dim) || !dtype_ok(dtype)) return GAT_ERR_UNSUPPORTED;
    if (n_rows == 0) return GAT_OK;
    if (!row_ptr || !out) return GAT_ERR_NULL;
    if (n_edges > 0 && (!col_idx || !weights || !feat)) return GAT_ERR_NULL;
    if (n_edges > 0 && n_src == 0) return GAT_ERR_ARGS;
    gat::PlanView pv;
    if (plan) {
        const gat_status st = check_plan(plan, row_ptr, n_rows, n_edges, (int64_t)heads * (head_dim + 2));
        if (st != GAT_OK) return st;
        pv = plan_view(plan);
    }
    return hip_status(gat::launch_spmm(gat::kAgg, dtype, heads, head_dim, row_ptr, col_idx, n_rows, n_src, weights,
                                       nullptr, nullptr, feat, 1.f, out, plan ? &pv : nullptr, stream));
}

// Argument checks of gat_fused_layer and its allocation-free variant (everything but the plan).
// GAT_OK with *nothing = true: no rows, nothing to enqueue.
gat_status check_fused(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t n_src,
                       int64_t n_edges, int heads, int head_dim, gat_dtype dtype, const float* scores, const void* q,
                       const void* k, const void* v, const float* out, bool* nothing) {
    *nothing = false;
    if (!size_ok(n_rows) || !size_ok(n_src) || !edges_ok(n_edges)) return GAT_ERR_SIZE;
    if (!shape_ok(heads, head_dim) || !dtype_ok(dtype)) return GAT_ERR_UNSUPPORTED;
    const bool have_scores = scores != nullptr;
    const bool have_q = q != nullptr, have_k = k != nullptr;
    // With no edges the output is +0.0 whatever the mode, and empty tensors carry NULL data pointers.
    if (n_edges > 0 && (have_q != have_k || have_scores == have_q)) return GAT_ERR_ARGS;
    if (n_rows == 0) {
        *nothing = true;
        return GAT_OK;
    }
    if (!row_ptr || !out) return GAT_ERR_NULL;
    if (n_edges > 0 && (!col_idx || !v)) return GAT_ERR_NULL;
    if (n_edges > 0 && n_src == 0) return GAT_ERR_ARGS;
    return GAT_OK;
}

gat_status gat_fused_layer(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t n_src,
                           int64_t n_edges, int heads, int head_dim, gat_dtype dtype, const float* scores,
                           const void* q, const void* k, float scale, const void* v, float* out,
                           const gat_plan* plan, hipStream_t stream) {
    bool nothing = false;
    const gat_status chk = check_fused(row_ptr, col_idx, n_rows, n_src, n_edges, heads, head_dim, dtype, scores, q,
                                       k, v, out, &nothing);
    if (chk != GAT_OK || nothing) return chk;
    const bool have_scores = scores != nullptr;
    gat::PlanView pv;
    if (plan) {
        const gat_status st = check_plan(plan, row_ptr, n_rows, n_edges, (int64_t)heads * (head_dim + 2));
        if (st != GAT_OK) return st;
        pv = plan_view(plan);
    }
    const int mode = have_scores ? gat::kSoftAgg : gat::kLayer;
    return hip_status(gat::launch_spmm(mode, dtype, heads, head_dim, row_ptr, col_idx, n_rows, n_src, scores, q, k, v,
                                       scale, out, plan ? &pv : nullptr, stream));
}

size_t gat_fused_layer_noalloc_bytes(int64_t n_rows, int64_t n_edges, int heads, int head_dim) {
    if (!size_ok(n_rows) || !edges_ok(n_edges) || !shape_ok(heads, head_dim)) return 0;
    return plan_layout(n_rows, n_edges, heads, head_dim, GAT_DEFAULT_SHORT_MAX, GAT_DEFAULT_SEG_LEN).total;
}

gat_status gat_fused_layer_noalloc(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t n_src,
                                   int64_t n_edges, int heads, int head_dim, gat_dtype dtype, const float* scores,
                                   const void* q, const void* k, float scale, const void* v, float* out,
                                   hipStream_t stream) {
    bool nothing = false;
    const gat_status chk = check_fused(row_ptr, col_idx, n_rows, n_src, n_edges, heads, head_dim, dtype, scores, q,
                                       k, v, out, &nothing);
    if (chk != GAT_OK || nothing) return chk;
    const Layout L = plan_layout(n_rows, n_edges, heads, head_dim, GAT_DEFAULT_SHORT_MAX, GAT_DEFAULT_SEG_LEN);
    if (L.total > (size_t)GAT_NOALLOC_SCRATCH_BYTES) return GAT_ERR_SCRATCH;
    void* ws = nullptr;   // the library's scratch array on this device
    if (gat::noalloc_scratch(&ws) != hipSuccess) return GAT_ERR_HIP;
    // Nothing in the plan's area must start at zero: the binner writes the counts, tables and
    // per-block sums it reads, and every hub partial is written before it is merged.
    gat_plan p;
    hipError_t e = build_plan(row_ptr, n_rows, n_edges, heads, head_dim, GAT_DEFAULT_SHORT_MAX, GAT_DEFAULT_SEG_LEN, L,
                              ws, (size_t)GAT_NOALLOC_SCRATCH_BYTES, &p, stream);
    if (e != hipSuccess) return GAT_ERR_HIP;
    const gat::PlanView pv = plan_view(&p);
    const int mode = scores != nullptr ? gat::kSoftAgg : gat::kLayer;
    return hip_status(gat::launch_spmm(mode, dtype, heads, head_dim, row_ptr, col_idx, n_rows, n_src, scores, q, k, v,
                                       scale, out, &pv, stream));
}

gat_status gat_batch_csr(const int32_t* local_row_ptr, const int32_t* local_col, const int32_t* row_off,
                         const int32_t* edge_off, const int32_t* src_off, int64_t n_graphs, int64_t n_rows,
                         int64_t n_edges, int32_t* row_ptr, int32_t* col_idx, hipStream_t stream) {
    if (n_graphs < 1 || n_graphs > kMaxIndex || !size_ok(n_rows) || !edges_ok(n_edges)) return GAT_ERR_SIZE;
    if (!local_row_ptr || !row_off || !edge_off || !row_ptr) return GAT_ERR_NULL;
    if (n_edges > 0 && (!local_col || !src_off || !col_idx)) return GAT_ERR_NULL;
    return hip_status(gat::launch_batch_csr(local_row_ptr, local_col, row_off, edge_off, src_off, n_graphs, n_rows,
                                            n_edges, row_ptr, col_idx, stream));
}

size_t gat_relation_block_lds_bytes(int n_nodes, int dim, int heads, int pair_dim) {
    if (n_nodes < 0 || n_nodes > 4096 || dim <= 0 || dim > gat::kRbMaxDim || heads <= 0 ||
        heads > gat::kRbMaxHeads || dim % heads != 0 || dim % 4 != 0 || pair_dim <= 0 || pair_dim > gat::kRbMaxPairDim)
        return 0;
    const size_t b = gat::relation_block_lds_bytes(n_nodes, dim, heads, pair_dim);
    return b <= gat::kRbMaxLds ? (b > 0 ? b : 1) : 0;
}

gat_status gat_relation_block(const float* nodes, const float* pair_feats, const float* edge_mask, const float* gamma,
                              const float* beta, float eps, const float* wq, const float* wk, const float* wv,
                              const float* wo, const float* w1, const float* b1, const float* w2, const float* b2,
                              int64_t batch, int n_nodes, int dim, int heads, int pair_dim, float* out,
                              hipStream_t stream) {
    if (batch < 0 || batch > kMaxIndex || n_nodes < 0 || n_nodes > 4096) return GAT_ERR_SIZE;
    if (gat_relation_block_lds_bytes(n_nodes, dim, heads, pair_dim) == 0) return GAT_ERR_UNSUPPORTED;
    if (batch == 0 || n_nodes == 0) return GAT_OK;
    if (!nodes || !pair_feats || !edge_mask || !gamma || !beta || !wq || !wk || !wv || !wo || !w1 || !b1 || !w2 ||
        !b2 || !out)
        return GAT_ERR_NULL;
    for (const float* p : {nodes, wq, wk, wv, wo, static_cast<const float*>(out)})
        if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return GAT_ERR_ARGS;   // 16-byte row loads
    return hip_status(gat::launch_relation_block(nodes, pair_feats, edge_mask, gamma, beta, eps, wq, wk, wv, wo, w1,
                                                 b1, w2, b2, batch, n_nodes, dim, heads, pair_dim, out, stream));
}

// ------------------------------------------------------------------------------ projections
gat_status gat_linear(const void* x, gat_dtype x_dtype, const uint16_t* w, const float* bias, int64_t n_rows,
                      int in_dim, int n_cols, void* const* out, int n_out, gat_dtype y_dtype,
                      hipStream_t stream) {
    if (!size_ok(n_rows)) return GAT_ERR_SIZE;
    if ((x_dtype != GAT_F32 && x_dtype != GAT_BF16) || (y_dtype != GAT_F32 && y_dtype != GAT_BF16) ||
        in_dim < 0 || in_dim > 65536 || in_dim % 8 != 0 || n_out < 1 || n_out > gat::kLinMaxOut || n_cols < 1 ||
        n_cols > 65536 || n_cols % n_out != 0)
        return GAT_ERR_UNSUPPORTED;
    const int64_t tiles = (n_rows + 127) / 128 * ((n_cols + 127) / 128);
    if (tiles > (int64_t{1} << 24)) return GAT_ERR_SIZE;       // grid of 256-thread workgroups
    if (out == nullptr) return GAT_ERR_NULL;
    if (n_rows == 0) return GAT_OK;                              // empty output arrays may be NULL
    gat::LinearOut o{};
    o.width = n_cols / n_out;
    for (int s = 0; s < n_out; ++s) {
        if (out[s] == nullptr) return GAT_ERR_NULL;
        o.p[s] = out[s];
    }
    if (in_dim > 0) {
        if (x == nullptr || w == nullptr) return GAT_ERR_NULL;
        if (reinterpret_cast<uintptr_t>(x) % 16 != 0 || reinterpret_cast<uintptr_t>(w) % 16 != 0) return GAT_ERR_ARGS;
    }
    return hip_status(gat::launch_linear(x, x_dtype == GAT_BF16, w, bias, n_rows, in_dim, n_cols, o,
                                         y_dtype == GAT_BF16, stream));
}

// ------------------------------------------------------------------------------ backward
size_t gat_csc_sizeof(void) { return sizeof(gat_csc); }

size_t gat_csc_workspace_bytes(int64_t n_rows, int64_t n_src, int64_t n_edges, int heads, int head_dim) {
    if (!size_ok(n_rows) || !size_ok(n_src) || !edges_ok(n_edges) || !shape_ok(heads, head_dim)) return 0;
    return csc_layout(n_rows, n_src, n_edges, heads, head_dim).total;
}

gat_status gat_csc_build(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t n_src,
                         int64_t n_edges, int heads, int head_dim, void* ws, size_t ws_bytes, gat_csc* csc,
                         hipStream_t stream) {
    if (csc == nullptr || ws == nullptr || row_ptr == nullptr) return GAT_ERR_NULL;
    if (!size_ok(n_rows) || !size_ok(n_src) || !edges_ok(n_edges)) return GAT_ERR_SIZE;
    if (!shape_ok(heads, head_dim)) return GAT_ERR_UNSUPPORTED;
    if (n_edges > 0 && (col_idx == nullptr || n_src == 0 || n_rows == 0)) return n_src == 0 || n_rows == 0 ? GAT_ERR_ARGS : GAT_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return GAT_ERR_ARGS;
    const CscLayout C = csc_layout(n_rows, n_src, n_edges, heads, head_dim);
    if (ws_bytes < C.total) return GAT_ERR_WORKSPACE;
    gat_csc c;
    memset(&c, 0, sizeof c);
    c.n_rows = n_rows;
    c.n_src = n_src;
    c.n_edges = n_edges;
    c.heads = heads;
    c.head_dim = head_dim;
    c.ws = ws;
    c.ws_bytes = ws_bytes;
    c.off_col_ptr = C.off_col_ptr;
    c.off_row_idx = C.off_row_idx;
    c.off_rows = C.off_rows;
    c.off_stage = C.off_stage;
    c.off_perm = C.off_vals[(C.sort.passes - 1) % 2];
    char* base = static_cast<char*>(ws);
    auto I = [&](size_t off) { return reinterpret_cast<int32_t*>(base + off); };
    hipError_t e = gat::launch_expand_rows(row_ptr, n_rows, I(C.off_rows), stream);
    // stable LSD passes over the column bits: (column, edge id) ends sorted by column, then edge id,
    // with each edge's row carried along (the last pass writes it into row_idx)
    const int np = C.sort.passes;
    auto rows_out = [&](int pass) { return I((np - 1 - pass) % 2 == 0 ? C.off_row_idx : C.off_rows2); };
    for (int pass = 0; e == hipSuccess && pass < np; ++pass) {
        const int32_t* kin = pass == 0 ? col_idx : I(C.off_keys[(pass - 1) % 2]);
        const int32_t* vin = pass == 0 ? nullptr : I(C.off_vals[(pass - 1) % 2]);
        const int32_t* rin = pass == 0 ? I(C.off_rows) : rows_out(pass - 1);
        e = gat::launch_radix_pass(kin, vin, I(C.off_keys[pass % 2]), I(C.off_vals[pass % 2]), rin, rows_out(pass),
                                   n_edges, pass * C.sort.bits, C.sort.bits, I(C.off_hist), I(C.off_sums), stream);
    }
    if (e == hipSuccess)
        e = gat::launch_bounds_from_keys(I(C.off_keys[(np - 1) % 2]), n_edges, n_src, I(C.off_col_ptr), stream);
    if (e == hipSuccess)
        e = build_plan(I(C.off_col_ptr), n_src, n_edges, heads, head_dim, GAT_DEFAULT_SHORT_MAX, GAT_DEFAULT_SEG_LEN,
                       C.plan, base + C.off_plan, C.plan.total, &c.plan, stream);
    if (e != hipSuccess) return GAT_ERR_HIP;
    c.magic = kCscMagic;
    *csc = c;
    return GAT_OK;
}

gat_status gat_edge_softmax_backward(const int32_t* row_ptr, int64_t n_rows, int64_t n_edges, int heads,
                                     const float* alpha, const float* grad, float* out, const gat_plan* plan,
                                     hipStream_t stream) {
    if (!size_ok(n_rows) || !edges_ok(n_edges)) return GAT_ERR_SIZE;
    if (!heads_ok(heads)) return GAT_ERR_UNSUPPORTED;
    if (n_rows == 0 || n_edges == 0) return GAT_OK;
    if (!row_ptr || !alpha || !grad || !out) return GAT_ERR_NULL;
    gat::PlanView pv;
    if (plan) {
        const gat_status st = check_plan(plan, row_ptr, n_rows, n_edges, heads);
        if (st != GAT_OK) return st;
        pv = plan_view(plan);
    }
    return hip_status(
        gat::launch_softmax_backward(heads, row_ptr, n_rows, alpha, grad, out, 1.f, plan ? &pv : nullptr, stream));
}

gat_status gat_aggregate_backward(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t n_src,
                                  int64_t n_edges, const float* weights, const void* feat, gat_dtype dtype, int heads,
                                  int head_dim, const float* grad_out, float* dweights, float* dfeat,
                                  const gat_csc* csc, hipStream_t stream) {
    if (!size_ok(n_rows) || !size_ok(n_src) || !edges_ok(n_edges)) return GAT_ERR_SIZE;
    if (!shape_ok(heads, head_dim) || !dtype_ok(dtype)) return GAT_ERR_UNSUPPORTED;
    if (csc == nullptr) return GAT_ERR_NULL;
    const gat_status st = check_csc(csc, n_rows, n_src, n_edges, heads, head_dim);
    if (st != GAT_OK) return st;
    if (n_edges > 0 && (!row_ptr || !col_idx || !grad_out)) return GAT_ERR_NULL;
    if (n_edges > 0 && dweights && !feat) return GAT_ERR_NULL;
    if (n_edges > 0 && dfeat && !weights) return GAT_ERR_NULL;
    hipError_t e = hipSuccess;
    if (dweights && n_edges > 0)
        e = gat::launch_edge_dot(dtype, heads, head_dim, at<int32_t>(csc, csc->off_rows), col_idx, n_edges, grad_out,
                                 feat, dweights, stream);
    if (e == hipSuccess && dfeat && n_src > 0) {
        const int32_t* perm = at<int32_t>(csc, csc->off_perm);
        float* stage = at<float>(csc, csc->off_stage);
        e = gat::launch_permute_edges(heads, perm, weights, n_edges, 1.f, stage, stream);
        const gat::PlanView pv = plan_view(&csc->plan);
        if (e == hipSuccess)
            e = gat::launch_spmm(gat::kAgg, GAT_F32, heads, head_dim, at<int32_t>(csc, csc->off_col_ptr),
                                 at<int32_t>(csc, csc->off_row_idx), n_src, n_rows, stage, nullptr, nullptr, grad_out,
                                 1.f, dfeat, &pv, stream);
    }
    return hip_status(e);
}

size_t gat_layer_backward_workspace_bytes(int64_t n_edges, int heads) {
    if (!edges_ok(n_edges) || !heads_ok(heads)) return 0;
    return bwd_layout(n_edges, heads).total;
}

gat_status gat_fused_layer_backward(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t n_src,
                                    int64_t n_edges, int heads, int head_dim, gat_dtype dtype, const float* scores,
                                    const void* q, const void* k, float scale, const void* v, const float* grad_out,
                                    float* dscores, float* dq, float* dk, float* dv, const gat_plan* plan,
                                    const gat_csc* csc, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!size_ok(n_rows) || !size_ok(n_src) || !edges_ok(n_edges)) return GAT_ERR_SIZE;
    if (!shape_ok(heads, head_dim) || !dtype_ok(dtype)) return GAT_ERR_UNSUPPORTED;
    const bool have_scores = scores != nullptr;
    const bool have_q = q != nullptr, have_k = k != nullptr;
    if (n_edges > 0 && (have_q != have_k || have_scores == have_q)) return GAT_ERR_ARGS;
    const bool layer = !have_scores && have_q;
    if (plan == nullptr || csc == nullptr || ws == nullptr) return GAT_ERR_NULL;
    gat_status st = check_plan(plan, row_ptr, n_rows, n_edges, (int64_t)heads * (head_dim + 2));
    if (st != GAT_OK) return st;
    st = check_csc(csc, n_rows, n_src, n_edges, heads, head_dim);
    if (st != GAT_OK) return st;
    if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return GAT_ERR_ARGS;
    const BwdLayout B = bwd_layout(n_edges, heads);
    if (ws_bytes < B.total) return GAT_ERR_WORKSPACE;
    if (n_src > 0 && !dv) return GAT_ERR_NULL;
    if (layer && ((n_rows > 0 && !dq) || (n_src > 0 && !dk))) return GAT_ERR_NULL;
    if (n_edges > 0 && (!row_ptr || !col_idx || !v || !grad_out)) return GAT_ERR_NULL;
    if (n_edges > 0 && !layer && !dscores) return GAT_ERR_NULL;
    char* base = static_cast<char*>(ws);
    float* s_ws = reinterpret_cast<float*>(base + B.off_scores);
    float* alpha = reinterpret_cast<float*>(base + B.off_alpha);
    float* g = reinterpret_cast<float*>(base + B.off_grad);
    const int32_t* rows = at<int32_t>(csc, csc->off_rows);
    const int32_t* perm = at<int32_t>(csc, csc->off_perm);
    const int32_t* col_ptr = at<int32_t>(csc, csc->off_col_ptr);
    const int32_t* row_idx = at<int32_t>(csc, csc->off_row_idx);
    float* stage = at<float>(csc, csc->off_stage);
    const gat::PlanView pv = plan_view(plan);
    const gat::PlanView cv = plan_view(&csc->plan);
    hipError_t e = hipSuccess;
    if (n_edges > 0) {
        const float* s = scores;
        if (layer) {   // the forward's scores, recomputed once
            e = gat::launch_sddmm(dtype, heads, head_dim, col_idx, rows, n_edges, k, n_src, q, n_rows, scale, s_ws,
                                  stream);
            s = s_ws;
        }
        // alpha, then dL/dalpha[e] = <grad_out[i], v[j]>, then the softmax backward (scaled for q, k)
        if (e == hipSuccess) e = gat::launch_softmax(heads, row_ptr, n_rows, s, alpha, &pv, stream);
        if (e == hipSuccess)
            e = gat::launch_edge_dot(dtype, heads, head_dim, rows, col_idx, n_edges, grad_out, v, g, stream);
        if (e == hipSuccess)
            e = gat::launch_softmax_backward(heads, row_ptr, n_rows, alpha, g, layer ? g : dscores,
                                             layer ? scale : 1.f, &pv, stream);
        if (e == hipSuccess) e = gat::launch_permute_edges(heads, perm, alpha, n_edges, 1.f, stage, stream);
    }
    // dv over the transposed graph (+0.0 for sources no edge reads)
    if (e == hipSuccess && n_src > 0)
        e = gat::launch_spmm(gat::kAgg, GAT_F32, heads, head_dim, col_ptr, row_idx, n_src, n_rows, stage, nullptr,
                             nullptr, grad_out, 1.f, dv, &cv, stream);
    if (layer) {
        if (e == hipSuccess && n_rows > 0)
            e = gat::launch_spmm(gat::kAgg, dtype, heads, head_dim, row_ptr, col_idx, n_rows, n_src, g, nullptr,
                                 nullptr, k, 1.f, dq, &pv, stream);
        if (e == hipSuccess && n_edges > 0)
            e = gat::launch_permute_edges(heads, perm, g, n_edges, 1.f, stage, stream);
        if (e == hipSuccess && n_src > 0)
            e = gat::launch_spmm(gat::kAgg, dtype, heads, head_dim, col_ptr, row_idx, n_src, n_rows, stage, nullptr,
                                 nullptr, q, 1.f, dk, &cv, stream);
    }
    return hip_status(e);
}

size_t gat_sddmm_backward_workspace_bytes(int64_t n_edges, int64_t n_src, int64_t n_dst, int heads, int head_dim) {
    if (!edges_ok(n_edges) || !size_ok(n_src) || !size_ok(n_dst) || !shape_ok(heads, head_dim)) return 0;
    return coo_bwd_layout(n_edges, n_src, n_dst, heads, head_dim).total;
}

gat_status gat_sddmm_backward(const int32_t* src_idx, const int32_t* dst_idx, int64_t n_edges, const void* src_feat,
                              int64_t n_src, const void* dst_feat, int64_t n_dst, gat_dtype dtype, int heads,
                              int head_dim, float scale, const float* grad_out, float* d_src, float* d_dst, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
    if (!edges_ok(n_edges) || !size_ok(n_src) || !size_ok(n_dst)) return GAT_ERR_SIZE;
    if (!shape_ok(heads, head_dim) || !dtype_ok(dtype)) return GAT_ERR_UNSUPPORTED;
    if (ws == nullptr) return GAT_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return GAT_ERR_ARGS;
    const CooBwdLayout C = coo_bwd_layout(n_edges, n_src, n_dst, heads, head_dim);
    if (ws_bytes < C.total) return GAT_ERR_WORKSPACE;
    if (n_edges > 0) {
        if (n_src == 0 || n_dst == 0) return GAT_ERR_ARGS;   // an edge needs a source and a destination row
        if (!src_idx || !dst_idx || !grad_out) return GAT_ERR_NULL;
        if ((d_src && !dst_feat) || (d_dst && !src_feat)) return GAT_ERR_NULL;
    }
    char* base = static_cast<char*>(ws);
    auto I = [&](size_t off) { return reinterpret_cast<int32_t*>(base + off); };
    int32_t* row_ptr = I(C.off_row_ptr);
    int32_t* col = I(C.off_col);
    float* w = reinterpret_cast<float*>(base + C.off_w);
    // side 0: d_dst, edges grouped by dst_idx, gathering src_feat; side 1: d_src, grouped by src_idx, gathering
    // dst_feat.  An output of a side with no rows, or not asked for, is skipped.
    struct Side {
        float* out;
        const int32_t* key;
        const int32_t* other;
        int64_t n_rows, n_other;
        const void* feat;
    };
    const Side sides[2] = {{d_dst, dst_idx, src_idx, n_dst, n_src, src_feat},
                           {d_src, src_idx, dst_idx, n_src, n_dst, dst_feat}};
    hipError_t e = hipSuccess;
    for (const Side& sd : sides) {
        if (sd.out == nullptr || sd.n_rows == 0) continue;
        // stable LSD passes over the key bits: (key, edge id) ends sorted by key, then edge id.  With no
        // edges the passes enqueue nothing, row_ptr is all zeros and the aggregation writes +0.0 rows.
        // (the other endpoint rides along; the last pass writes it into col)
        const gat::RadixPlan rp = gat::radix_plan(sd.n_rows);
        const int np = rp.passes;
        auto other_out = [&](int pass) { return I((np - 1 - pass) % 2 == 0 ? C.off_col : C.off_col2); };
        for (int pass = 0; e == hipSuccess && pass < np; ++pass) {
            const int32_t* kin = pass == 0 ? sd.key : I(C.off_keys[(pass - 1) % 2]);
            const int32_t* vin = pass == 0 ? nullptr : I(C.off_vals[(pass - 1) % 2]);
            const int32_t* oin = pass == 0 ? sd.other : other_out(pass - 1);
            e = gat::launch_radix_pass(kin, vin, I(C.off_keys[pass % 2]), I(C.off_vals[pass % 2]), oin,
                                       other_out(pass), n_edges, pass * rp.bits, rp.bits, I(C.off_hist),
                                       I(C.off_sums), stream);
        }
        const int32_t* perm = I(C.off_vals[(np - 1) % 2]);
        if (e == hipSuccess)
            e = gat::launch_bounds_from_keys(I(C.off_keys[(np - 1) % 2]), n_edges, sd.n_rows, row_ptr, stream);
        // the scaled gradient in the grouping's order
        if (e == hipSuccess) e = gat::launch_permute_edges(heads, perm, grad_out, n_edges, scale, w, stream);
        gat_plan plan;
        const Layout L =
            plan_layout(sd.n_rows, n_edges, heads, head_dim, GAT_DEFAULT_SHORT_MAX, GAT_DEFAULT_SEG_LEN);
        if (e == hipSuccess)
            e = build_plan(row_ptr, sd.n_rows, n_edges, heads, head_dim, GAT_DEFAULT_SHORT_MAX, GAT_DEFAULT_SEG_LEN, L,
                           base + C.off_plan, C.plan_bytes, &plan, stream);
        if (e == hipSuccess) {
            const gat::PlanView pv = plan_view(&plan);
            e = gat::launch_spmm(gat::kAgg, dtype, heads, head_dim, row_ptr, col, sd.n_rows, sd.n_other, w, nullptr,
                                 nullptr, sd.feat, 1.f, sd.out, &pv, stream);
        }
        if (e != hipSuccess) break;
    }
    return hip_status(e);
}

}  // extern "C"
