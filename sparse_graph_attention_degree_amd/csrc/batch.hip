// A batch of CSR graphs as one block-diagonal CSR.
//
// Small graphs (the 384-node problem of POPCORNBENCH l2_p37, whose work the page finds too small
// for the launch overhead) are launch-bound one at a time.  Stacked block-diagonally -- rows,
// edges and sources of graph b shifted by the totals of graphs 0..b-1 -- any number of them is one
// graph, and every entry point then covers the whole batch in the launches of a single call.  Each
// row's arithmetic is unchanged (a row only ever meets its own edges), so batched outputs equal
// the per-graph outputs bit for bit.
//
// One thread per global row writes row_ptr, one per global edge writes col_idx; the graph of an
// item is found by binary search over the batch's offsets.
#include "kernels.hpp"

namespace gat {

namespace {

// largest b in [0, n) with off[b] <= x (off non-decreasing, off[0] = 0 <= x)
__device__ __forceinline__ int64_t graph_of(const int32_t* __restrict__ off, int64_t n, int64_t x) {
    int64_t lo = 0, hi = n;   // off[lo] <= x, answer in [lo, hi)
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) / 2;
        if (off[mid] <= x) lo = mid;
        else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(kBlock) void batch_rows_kernel(const int32_t* __restrict__ local_row_ptr,
                                                            const int32_t* __restrict__ row_off,
                                                            const int32_t* __restrict__ edge_off, int64_t n_graphs,
                                                            int64_t n_rows, int64_t n_edges,
                                                            int32_t* __restrict__ row_ptr) {
    for (int64_t r = (int64_t)blockIdx.x * kBlock + threadIdx.x; r <= n_rows; r += (int64_t)gridDim.x * kBlock) {
        if (r == n_rows) {
            row_ptr[r] = (int32_t)n_edges;
            continue;
        }
        // graphs without rows share their offset with the next graph: take the last such b
        const int64_t b = graph_of(row_off, n_graphs, r);
        row_ptr[r] = edge_off[b] + local_row_ptr[r + b];
    }
}

__global__ __launch_bounds__(kBlock) void batch_cols_kernel(const int32_t* __restrict__ local_col,
                                                            const int32_t* __restrict__ edge_off,
                                                            const int32_t* __restrict__ src_off, int64_t n_graphs,
                                                            int64_t n_edges, int32_t* __restrict__ col) {
    for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < n_edges; e += (int64_t)gridDim.x * kBlock)
        col[e] = src_off[graph_of(edge_off, n_graphs, e)] + local_col[e];
}

}  // namespace

hipError_t launch_batch_csr(const int32_t* local_row_ptr, const int32_t* local_col, const int32_t* row_off,
                            const int32_t* edge_off, const int32_t* src_off, int64_t n_graphs, int64_t n_rows,
                            int64_t n_edges, int32_t* row_ptr, int32_t* col, hipStream_t stream) {
    hipLaunchKernelGGL(batch_rows_kernel, dim3(grid_for(n_rows + 1, kBlock, 65536)), dim3(kBlock), 0, stream,
                       local_row_ptr, row_off, edge_off, n_graphs, n_rows, n_edges, row_ptr);
    if (n_edges > 0)
        hipLaunchKernelGGL(batch_cols_kernel, dim3(grid_for(n_edges, kBlock, 65536)), dim3(kBlock), 0, stream,
                           local_col, edge_off, src_off, n_graphs, n_edges, col);
    return hipGetLastError();
}

}  // namespace gat
