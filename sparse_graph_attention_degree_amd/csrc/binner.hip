// Degree binning on the device.
//
// The pages size per-row work from a maximum degree that the host computes after
// copying row_ptr back (POPCORNBENCH l2_p37, the passages on max_degree and the
// device-to-host copy that synchronises the GPU).  Here every row is classified
// by its own degree instead, on the device, with no host round trip:
//   short  deg <= short_max              -> lane-group kernels (no table entry)
//   long   short_max < deg <= seg_len    -> one segment = the whole row
//   hub    deg > both                    -> ceil(deg / seg_len) segments
// Three kernels build a stable counting sort: per-block counts, one-block
// exclusive scan, then a scatter that recomputes the classes and writes the
// segment table (hub segments first, then long rows) and the hub table.
#include "kernels.hpp"

namespace gat {

namespace {

struct Triple {
    int a, b, c;   // long rows, hub rows, hub segments
};

__device__ __forceinline__ Triple add(Triple x, Triple y) { return {x.a + y.a, x.b + y.b, x.c + y.c}; }

__device__ __forceinline__ void classify(int deg, int short_max, int seg_len, int& is_long, int& is_hub,
                                         int& nseg) {
    is_long = 0;
    is_hub = 0;
    nseg = 0;
    if (deg <= short_max) return;
    if (deg <= seg_len) {
        is_long = 1;
        return;
    }
    is_hub = 1;
    nseg = (int)(((int64_t)deg + seg_len - 1) / seg_len);
}

// Block-wide exclusive scan of one Triple per thread; `total` gets the block sum.
__device__ Triple block_exscan(Triple v, Triple& total) {
    __shared__ Triple wave_sum[kWavesPerBlock];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    Triple inc = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int a = __shfl_up(inc.a, o), b = __shfl_up(inc.b, o), c = __shfl_up(inc.c, o);
        if (lane >= o) {
            inc.a += a;
            inc.b += b;
            inc.c += c;
        }
    }
    if (lane == kWave - 1) wave_sum[w] = inc;
    __syncthreads();
    Triple off = {0, 0, 0};
    total = {0, 0, 0};
#pragma unroll
    for (int i = 0; i < kWavesPerBlock; ++i) {
        if (i < w) off = add(off, wave_sum[i]);
        total = add(total, wave_sum[i]);
    }
    __syncthreads();
    return {off.a + inc.a - v.a, off.b + inc.b - v.b, off.c + inc.c - v.c};
}

__global__ __launch_bounds__(kBlock) void plan_count_kernel(const int32_t* __restrict__ row_ptr,
                                                            int64_t n_rows, int short_max, int seg_len,
                                                            int4* __restrict__ blocks) {
    const int64_t r0 = (int64_t)blockIdx.x * kPlanRowsPerBlock + (int64_t)threadIdx.x * kPlanRowsPerThread;
    Triple c = {0, 0, 0};
#pragma unroll
    for (int k = 0; k < kPlanRowsPerThread; ++k) {
        const int64_t r = r0 + k;
        if (r < n_rows) {
            int is_long, is_hub, nseg;
            classify(row_ptr[r + 1] - row_ptr[r], short_max, seg_len, is_long, is_hub, nseg);
            c = add(c, Triple{is_long, is_hub, nseg});
        }
    }
    Triple tot;
    block_exscan(c, tot);
    if (threadIdx.x == 0) blocks[blockIdx.x] = make_int4(tot.a, tot.b, tot.c, 0);
}

// One workgroup: exclusive scan of the per-block counts (in place) and the totals.  Totals past
// the table capacities (a row_ptr whose degrees sum past n_edges) set the overflow flag and
// leave every table empty, so no kernel reads or writes past the workspace.
__global__ __launch_bounds__(kBlock) void plan_scan_kernel(int4* __restrict__ blocks, int64_t n_blocks,
                                                           int32_t* __restrict__ counts, PlanCaps caps) {
    Triple carry = {0, 0, 0};
    for (int64_t base = 0; base < n_blocks; base += kBlock) {
        const int64_t i = base + threadIdx.x;
        Triple v = {0, 0, 0};
        if (i < n_blocks) {
            int4 b = blocks[i];
            v = {b.x, b.y, b.z};
        }
        Triple tot;
        Triple ex = block_exscan(v, tot);
        if (i < n_blocks) blocks[i] = make_int4(carry.a + ex.a, carry.b + ex.b, carry.c + ex.c, 0);
        carry = add(carry, tot);
    }
    if (threadIdx.x == 0) {
        const bool over = (int64_t)carry.c + carry.a > caps.segs || carry.b > caps.hubs || carry.c > caps.hub_segs ||
                          carry.a < 0 || carry.b < 0 || carry.c < 0;
        counts[kNSegs] = over ? 0 : carry.c + carry.a;
        counts[kNHubSegs] = over ? 0 : carry.c;
        counts[kNHubs] = over ? 0 : carry.b;
        counts[kNLong] = over ? 0 : carry.a;
        counts[kOverflow] = over ? 1 : 0;
    }
}

__global__ __launch_bounds__(kBlock) void plan_scatter_kernel(const int32_t* __restrict__ row_ptr,
                                                              int64_t n_rows, int short_max, int seg_len,
                                                              const int4* __restrict__ blocks,
                                                              const int32_t* __restrict__ counts,
                                                              int4* __restrict__ segs, int4* __restrict__ hubs) {
    const int64_t r0 = (int64_t)blockIdx.x * kPlanRowsPerBlock + (int64_t)threadIdx.x * kPlanRowsPerThread;
    int e0[kPlanRowsPerThread], e1[kPlanRowsPerThread], il[kPlanRowsPerThread], ih[kPlanRowsPerThread],
        ns[kPlanRowsPerThread];
    Triple c = {0, 0, 0};
#pragma unroll
    for (int k = 0; k < kPlanRowsPerThread; ++k) {
        const int64_t r = r0 + k;
        e0[k] = e1[k] = il[k] = ih[k] = ns[k] = 0;
        if (r < n_rows) {
            e0[k] = row_ptr[r];
            e1[k] = row_ptr[r + 1];
            classify(e1[k] - e0[k], short_max, seg_len, il[k], ih[k], ns[k]);
            c = add(c, Triple{il[k], ih[k], ns[k]});
        }
    }
    Triple tot;
    const Triple ex = block_exscan(c, tot);
    if (counts[kOverflow]) return;   // the tables stay empty
    const int4 base = blocks[blockIdx.x];
    const int n_hub_segs = counts[kNHubSegs];
    int pos_long = base.x + ex.a, pos_hub = base.y + ex.b, pos_hs = base.z + ex.c;
#pragma unroll
    for (int k = 0; k < kPlanRowsPerThread; ++k) {
        const int row = (int)(r0 + k);
        if (il[k]) segs[n_hub_segs + pos_long++] = make_int4(row, e0[k], e1[k], -1);
        if (ih[k]) {
            hubs[pos_hub++] = make_int4(row, pos_hs, ns[k], 0);
            for (int j = 0; j < ns[k]; ++j) {
                const int64_t b = (int64_t)e0[k] + (int64_t)j * seg_len;
                const int64_t e = b + seg_len < (int64_t)e1[k] ? b + seg_len : (int64_t)e1[k];
                segs[pos_hs + j] = make_int4(row, (int)b, (int)e, pos_hs + j);
            }
            pos_hs += ns[k];
        }
    }
}

}  // namespace

hipError_t launch_plan(const int32_t* row_ptr, int64_t n_rows, int short_max, int seg_len, int4* blocks,
                       int64_t n_blocks, int32_t* counts, int4* segs, int4* hubs, PlanCaps caps,
                       hipStream_t stream) {
    if (n_blocks > 0)
        hipLaunchKernelGGL(plan_count_kernel, dim3((unsigned)n_blocks), dim3(kBlock), 0, stream, row_ptr, n_rows,
                           short_max, seg_len, blocks);
    hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(kBlock), 0, stream, blocks, n_blocks, counts, caps);
    if (n_blocks > 0)
        hipLaunchKernelGGL(plan_scatter_kernel, dim3((unsigned)n_blocks), dim3(kBlock), 0, stream, row_ptr,
                           n_rows, short_max, seg_len, blocks, counts, segs, hubs);
    return hipGetLastError();
}

}  // namespace gat
