// Host-side launch entry points of the gfx950 kernels (one per .hip file) and the
// compile-time shape dispatch they share.  Everything here is internal to
// libgat.so; the public interface is include/gat.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace gat {

enum SpmmMode { kAgg = 0, kSoftAgg = 1, kLayer = 2 };

// ---------------------------------------------------------------------------- dispatch
template <typename T, int H_, int D_>
struct ShapeTag {
    using type = T;
    static constexpr int H = H_;
    static constexpr int D = D_;
};

template <int H, int D, typename F>
bool dispatch_dtype(int dtype, F&& f) {
    if constexpr (H * D <= 1024) {
        if (dtype == 0) { f(ShapeTag<float, H, D>{}); return true; }
        if (dtype == 1) { f(ShapeTag<bf16_t, H, D>{}); return true; }
    }
    return false;
}

template <int H, typename F>
bool dispatch_dim(int dtype, int D, F&& f) {
    switch (D) {
        case 16: return dispatch_dtype<H, 16>(dtype, f);
        case 32: return dispatch_dtype<H, 32>(dtype, f);
        case 64: return dispatch_dtype<H, 64>(dtype, f);
        case 128: return dispatch_dtype<H, 128>(dtype, f);
        default: return false;
    }
}

// Calls f(ShapeTag<T, H, D>{}) for a supported (dtype, H, D); returns false otherwise.
template <typename F>
bool dispatch_shape(int dtype, int H, int D, F&& f) {
    switch (H) {
        case 1: return dispatch_dim<1>(dtype, D, f);
        case 2: return dispatch_dim<2>(dtype, D, f);
        case 4: return dispatch_dim<4>(dtype, D, f);
        case 8: return dispatch_dim<8>(dtype, D, f);
        case 16: return dispatch_dim<16>(dtype, D, f);
        default: return false;
    }
}

template <class T>
struct TypeTag {
    using type = T;
};

template <typename F>
bool dispatch_heads(int H, F&& f) {
    switch (H) {
        case 1: f(ShapeTag<float, 1, 0>{}); return true;
        case 2: f(ShapeTag<float, 2, 0>{}); return true;
        case 4: f(ShapeTag<float, 4, 0>{}); return true;
        case 8: f(ShapeTag<float, 8, 0>{}); return true;
        case 16: f(ShapeTag<float, 16, 0>{}); return true;
        default: return false;
    }
}

inline unsigned grid_for(int64_t items, int64_t per_block, int64_t cap) {
    int64_t g = (items + per_block - 1) / per_block;
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    return (unsigned)g;
}

// ---------------------------------------------------------------------------- launchers
// Every launcher enqueues on `stream` and returns hipGetLastError() (hipErrorInvalidValue
// for an unsupported shape, which the C-ABI has already ruled out).

// capacities of the plan's tables (entries)
struct PlanCaps {
    int64_t segs, hubs, hub_segs;
};

hipError_t launch_plan(const int32_t* row_ptr, int64_t n_rows, int short_max, int seg_len,
                       int4* blocks, int64_t n_blocks, int32_t* counts, int4* segs, int4* hubs,
                       PlanCaps caps, hipStream_t stream);

hipError_t launch_sddmm(int dtype, int H, int D, const int32_t* src_idx, const int32_t* dst_idx,
                        int64_t n_edges, const void* src_feat, int64_t n_src, const void* dst_feat,
                        int64_t n_dst, float scale, float* out, hipStream_t stream);

hipError_t launch_softmax(int H, const int32_t* row_ptr, int64_t n_rows, const float* scores,
                          float* out, const PlanView* plan, hipStream_t stream);

// mode kAgg: weights in `scores`; kSoftAgg: scores; kLayer: q, k (scores unused).
hipError_t launch_spmm(int mode, int dtype, int H, int D, const int32_t* row_ptr, const int32_t* col_idx,
                       int64_t n_rows, int64_t n_src, const float* scores, const void* q, const void* k, const void* v,
                       float scale, float* out, const PlanView* plan, hipStream_t stream);

// ---------------------------------------------------------------------------- backward
hipError_t launch_expand_rows(const int32_t* row_ptr, int64_t n_rows, int32_t* rows, hipStream_t stream);

// radix sort of (column, edge id): tiles per pass, and tiles of the scan of the digit counts
int64_t radix_tiles(int64_t n);
int64_t scan_tiles(int64_t n);
constexpr int kRadixMaxBits = 8;
constexpr int kRadixMaxBins = 1 << kRadixMaxBits;

// LSD passes for keys in [0, n_keys): `passes` digits of `bits` bits each (bits <= 8, as even as
// possible; one 1-bit pass for n_keys <= 1).
struct RadixPlan {
    int passes, bits;
};
RadixPlan radix_plan(int64_t n_keys);

// one stable pass on bits [shift, shift+bits) of the keys; vin == nullptr means values = positions.
// v2in / v2out (both or neither): a second value carried with each key.
// hist: int32 [256 * radix_tiles(n)], sums: int32 [scan_tiles(256 * radix_tiles(n)) + 1].
hipError_t launch_radix_pass(const int32_t* kin, const int32_t* vin, int32_t* kout, int32_t* vout,
                             const int32_t* v2in, int32_t* v2out, int64_t n, int shift, int bits, int32_t* hist,
                             int32_t* sums, hipStream_t stream);

// row_ptr [n_rows+1] of the grouping from the sorted keys (< n_rows)
hipError_t launch_bounds_from_keys(const int32_t* skeys, int64_t n_edges, int64_t n_rows, int32_t* row_ptr,
                                   hipStream_t stream);

// dst[p,:] = scale * src[perm[p],:], [E,H] fp32
hipError_t launch_permute_edges(int H, const int32_t* perm, const float* src, int64_t n, float scale, float* dst,
                                hipStream_t stream);

// out[e,h] = <G[rows[e],h,:], F[col[e],h,:]>, G fp32 [*,H,D], F of dtype
hipError_t launch_edge_dot(int dtype, int H, int D, const int32_t* rows, const int32_t* col, int64_t n_edges,
                           const float* gf, const void* ff, float* out, hipStream_t stream);

// out = scale * alpha * (grad - sum_row alpha * grad)
hipError_t launch_softmax_backward(int H, const int32_t* row_ptr, int64_t n_rows, const float* alpha,
                                   const float* grad, float* out, float scale, const PlanView* plan,
                                   hipStream_t stream);

// block-diagonal batch of CSR graphs (offsets: device int32 [n_graphs+1] prefix sums)
hipError_t launch_batch_csr(const int32_t* local_row_ptr, const int32_t* local_col, const int32_t* row_off,
                            const int32_t* edge_off, const int32_t* src_off, int64_t n_graphs, int64_t n_rows,
                            int64_t n_edges, int32_t* row_ptr, int32_t* col, hipStream_t stream);

// dense relation-biased attention block: one workgroup per batch element, everything in LDS
constexpr size_t kRbMaxLds = 160 * 1024;   // gfx950 LDS per workgroup
constexpr int kRbMaxHeads = 16;
size_t relation_block_lds_bytes(int N, int D, int H, int P);
constexpr int kRbMaxPairDim = 64;
constexpr int kRbMaxDim = 256;   // a block of 16 weight rows is at most 4 float4 loads per thread
hipError_t launch_relation_block(const float* nodes, const float* pair, const float* mask, const float* gamma,
                                 const float* beta, float eps, const float* wq, const float* wk, const float* wv,
                                 const float* wo, const float* w1, const float* b1, const float* w2, const float* b2,
                                 int64_t B, int N, int D, int H, int P, float* out, hipStream_t stream);

// Device address of the library's own scratch array on the current device (looked up on the
// first call per device), for the entry point that allocates nothing.
hipError_t noalloc_scratch(void** addr);

// Rows per binner block (256 threads x 4 consecutive rows).
constexpr int kPlanRowsPerThread = 4;
constexpr int kPlanRowsPerBlock = kBlock * kPlanRowsPerThread;

}  // namespace gat
