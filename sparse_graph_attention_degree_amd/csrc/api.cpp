// C-ABI of libgat.so (declared in include/gat.h): host-side argument checks, plan
// layout, and dispatch to the gfx950 kernels.  Every check runs before anything is
// enqueued; no exception leaves this file.
#include "gat.h"

#include <limits.h>
#include <string.h>

#include "kernels.hpp"

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

// A plan usable for a call on (n_rows, n_edges) needing `floats` floats of state per hub segment.
gat_status check_plan(const gat_plan* p, int64_t n_rows, int64_t n_edges, int64_t floats) {
    if (p->magic != kPlanMagic || p->ws == nullptr) return GAT_ERR_ARGS;
    if (p->n_rows != n_rows || p->n_edges != n_edges) return GAT_ERR_WORKSPACE;
    if (floats > p->state_floats) return GAT_ERR_WORKSPACE;
    return GAT_OK;
}

gat_status hip_status(hipError_t e) { return e == hipSuccess ? GAT_OK : GAT_ERR_HIP; }

}  // namespace

extern "C" {

const char* gat_status_str(gat_status s) {
    switch (s) {
        case GAT_OK: return "ok";
        case GAT_ERR_NULL: return "required pointer is NULL";
        case GAT_ERR_SIZE: return "size negative or above INT32_MAX";
        case GAT_ERR_UNSUPPORTED: return "unsupported heads/head_dim/dtype";
        case GAT_ERR_WORKSPACE: return "plan workspace too small or built for other sizes";
        case GAT_ERR_ARGS: return "inconsistent arguments";
        case GAT_ERR_HIP: return "HIP launch or runtime error";
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
    memset(&p, 0, sizeof p);
    p.n_rows = n_rows;
    p.n_edges = n_edges;
    p.short_max = short_max;
    p.seg_len = seg_len;
    p.heads = heads;
    p.head_dim = head_dim;
    p.state_floats = L.state_floats;
    p.seg_capacity = L.seg_cap;
    p.hub_capacity = L.hub_cap;
    p.hubseg_capacity = L.hubseg_cap;
    p.n_blocks = L.n_blocks;
    p.ws = ws;
    p.ws_bytes = ws_bytes;
    p.off_counts = L.off_counts;
    p.off_blocks = L.off_blocks;
    p.off_segs = L.off_segs;
    p.off_hubs = L.off_hubs;
    p.off_partials = L.off_partials;
    p.magic = kPlanMagic;
    char* base = static_cast<char*>(ws);
    const hipError_t e = gat::launch_plan(row_ptr, n_rows, short_max, seg_len,
                                          reinterpret_cast<int4*>(base + L.off_blocks), L.n_blocks,
                                          reinterpret_cast<int32_t*>(base + L.off_counts),
                                          reinterpret_cast<int4*>(base + L.off_segs),
                                          reinterpret_cast<int4*>(base + L.off_hubs), stream);
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
        const gat_status st = check_plan(plan, n_rows, n_edges, 2 * (int64_t)heads);
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
        const gat_status st = check_plan(plan, n_rows, n_edges, (int64_t)heads * (head_dim + 2));
        if (st != GAT_OK) return st;
        pv = plan_view(plan);
    }
    return hip_status(gat::launch_spmm(gat::kAgg, dtype, heads, head_dim, row_ptr, col_idx, n_rows, n_src, weights,
                                       nullptr, nullptr, feat, 1.f, out, plan ? &pv : nullptr, stream));
}

gat_status gat_fused_layer(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t n_src,
                           int64_t n_edges, int heads, int head_dim, gat_dtype dtype, const float* scores,
                           const void* q, const void* k, float scale, const void* v, float* out,
                           const gat_plan* plan, hipStream_t stream) {
    if (!size_ok(n_rows) || !size_ok(n_src) || !edges_ok(n_edges)) return GAT_ERR_SIZE;
    if (!shape_ok(heads, head_dim) || !dtype_ok(dtype)) return GAT_ERR_UNSUPPORTED;
    const bool have_scores = scores != nullptr;
    const bool have_q = q != nullptr, have_k = k != nullptr;
    // With no edges the output is +0.0 whatever the mode, and empty tensors carry NULL data pointers.
    if (n_edges > 0 && (have_q != have_k || have_scores == have_q)) return GAT_ERR_ARGS;
    if (n_rows == 0) return GAT_OK;
    if (!row_ptr || !out) return GAT_ERR_NULL;
    if (n_edges > 0 && (!col_idx || !v)) return GAT_ERR_NULL;
    if (n_edges > 0 && n_src == 0) return GAT_ERR_ARGS;
    gat::PlanView pv;
    if (plan) {
        const gat_status st = check_plan(plan, n_rows, n_edges, (int64_t)heads * (head_dim + 2));
        if (st != GAT_OK) return st;
        pv = plan_view(plan);
    }
    const int mode = have_scores ? gat::kSoftAgg : gat::kLayer;
    return hip_status(gat::launch_spmm(mode, dtype, heads, head_dim, row_ptr, col_idx, n_rows, n_src, scores, q, k, v,
                                       scale, out, plan ? &pv : nullptr, stream));
}

}  // extern "C"
