// Row-wise multi-head edge softmax (POPCORNBENCH l1_p6, the reference model: for
// every node and head, softmax over the node's edge slice of scores [E,H],
// computed as exp(x - max) / sum(exp(x - max))).
//
// The page's kernels map one thread to a (node, head) pair striding through the
// slice with stride H, or one block per node with shared-memory reductions.
// Here the [E,H] slice of a row is contiguous, so a 32-lane slot reads it 32
// values at a time with coalesced dword loads (lane q: edge q/H, head q%H) and
// the per-head max / sum are xor-shuffle trees over lanes q, q^H, q^2H, ...
// Three passes over the row: max, sum of exp, write.  Degree binning splits long
// rows over a workgroup and hub rows over segments whose (max, sum) states merge.
#include <math.h>

#include "kernels.hpp"

namespace gat {

namespace {

constexpr int kSmG = 32;                       // lanes per row slot
constexpr int kSmP = kWave / kSmG;             // rows per wave step
constexpr int kSmRowsPerWave = 32;

template <int H>
struct SmSlot {
    static constexpr int SC = kSmG / H;        // edges per chunk
    int q;

    __device__ __forceinline__ void stats(const float* __restrict__ sc, int e0, int e1, float& m, float& z) const {
        const int es = q / H;
        m = -INFINITY;
        for (int c = e0; c < e1; c += SC)
            if (c + es < e1) m = fmaxf(m, sc[(int64_t)c * H + q]);
#pragma unroll
        for (int k = H; k < kSmG; k <<= 1) m = fmaxf(m, shfl_xor(m, k));
        z = 0.f;
        for (int c = e0; c < e1; c += SC)
            if (c + es < e1) z += exp_fast(sc[(int64_t)c * H + q] - m);
#pragma unroll
        for (int k = H; k < kSmG; k <<= 1) z += shfl_xor(z, k);
    }

    // alpha = exp(s - m) / z over [e0, e1); m, z in score layout (lane q: head q % H)
    __device__ __forceinline__ void write(const float* sc, float* out, int e0, int e1, float m, float z) const {
        const int es = q / H;
        for (int c = e0; c < e1; c += SC)
            if (c + es < e1) {
                const int64_t i = (int64_t)c * H + q;
                out[i] = exp_fast(sc[i] - m) / z;
            }
    }
};

template <int H>
__global__ __launch_bounds__(kBlock) void softmax_short_kernel(const int32_t* __restrict__ row_ptr, int64_t n_rows,
                                                               const float* sc, float* out, int short_max) {
    const int lane = lane_id();
    const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    const int64_t wb = wave * kSmRowsPerWave;
    if (wb >= n_rows) return;
    int rpv = 0;
    if (lane <= kSmRowsPerWave && wb + lane <= n_rows) rpv = row_ptr[wb + lane];
    SmSlot<H> sl;
    sl.q = lane % kSmG;
    const int g = lane / kSmG;
#pragma unroll 1
    for (int it = 0; it < kSmRowsPerWave / kSmP; ++it) {
        const int j = it * kSmP + g;
        int e0 = shfl(rpv, j), e1 = shfl(rpv, j + 1);
        if (!(wb + j < n_rows && e1 - e0 <= short_max)) e1 = e0;
        float m, z;
        sl.stats(sc, e0, e1, m, z);
        sl.write(sc, out, e0, e1, m, z);
    }
}

// One workgroup per plan segment; 8 slots split it.  Long rows are written here; hub
// segments leave (max[H], sum[H]) in the partial buffer.
template <int H>
__global__ __launch_bounds__(kBlock) void softmax_segment_kernel(const float* sc, float* out, PlanView plan) {
    constexpr int NS = kBlock / kSmG;
    __shared__ float lm[NS][H], lz[NS][H], gm[H], gz[H];
    const int lane = lane_id();
    const int gs = threadIdx.x / kSmG;
    SmSlot<H> sl;
    sl.q = lane % kSmG;
    const int n_segs = plan.counts[kNSegs];
    for (int s = blockIdx.x; s < n_segs; s += gridDim.x) {
        const int4 sg = plan.segs[s];
        const int64_t len = (int64_t)sg.z - sg.y;
        const int b = sg.y + (int)(len * gs / NS), e = sg.y + (int)(len * (gs + 1) / NS);
        float m, z;
        sl.stats(sc, b, e, m, z);
        if (sl.q < H) {
            lm[gs][sl.q] = m;
            lz[gs][sl.q] = z;
        }
        __syncthreads();
        if (threadIdx.x < H) {
            const int h = threadIdx.x;
            float M = -INFINITY, Z = 0.f;
            for (int i = 0; i < NS; ++i) M = fmaxf(M, lm[i][h]);
            for (int i = 0; i < NS; ++i)
                if (lm[i][h] != -INFINITY) Z = fmaf(lz[i][h], exp_fast(lm[i][h] - M), Z);
            gm[h] = M;
            gz[h] = Z;
            if (sg.w >= 0) {
                float* prt = plan.partials + (int64_t)sg.w * plan.state_floats;
                prt[h] = M;
                prt[H + h] = Z;
            }
        }
        __syncthreads();
        if (sg.w < 0) sl.write(sc, out, b, e, gm[sl.q % H], gz[sl.q % H]);
        __syncthreads();
    }
}

// One workgroup per hub segment: merge the row's segment states, then write alpha.
template <int H>
__global__ __launch_bounds__(kBlock) void softmax_hub_write_kernel(const int32_t* __restrict__ row_ptr,
                                                                   const float* sc, float* out, PlanView plan) {
    __shared__ float gm[H], gz[H];
    const int n_hub_segs = plan.counts[kNHubSegs];
    for (int s = blockIdx.x; s < n_hub_segs; s += gridDim.x) {
        const int4 sg = plan.segs[s];   // row, b, e, slot (= s)
        const int rb = row_ptr[sg.x], re = row_ptr[sg.x + 1];
        const int first = sg.w - (int)(((int64_t)sg.y - rb) / plan.seg_len);
        const int nseg = (int)(((int64_t)re - rb + plan.seg_len - 1) / plan.seg_len);
        if (threadIdx.x < H) {
            const int h = threadIdx.x;
            const float* p0 = plan.partials + (int64_t)first * plan.state_floats;
            float M = -INFINITY, Z = 0.f;
            for (int c = 0; c < nseg; ++c) M = fmaxf(M, p0[(int64_t)c * plan.state_floats + h]);
            for (int c = 0; c < nseg; ++c) {
                const float* pc = p0 + (int64_t)c * plan.state_floats;
                if (pc[h] != -INFINITY) Z = fmaf(pc[H + h], exp_fast(pc[h] - M), Z);
            }
            gm[h] = M;
            gz[h] = Z;
        }
        __syncthreads();
        for (int64_t i = (int64_t)sg.y * H + threadIdx.x; i < (int64_t)sg.z * H; i += kBlock) {
            const int h = (int)(i % H);
            out[i] = exp_fast(sc[i] - gm[h]) / gz[h];
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_softmax(int H, const int32_t* row_ptr, int64_t n_rows, const float* scores, float* out,
                          const PlanView* plan, hipStream_t stream) {
    const bool ok = dispatch_heads(H, [&](auto tag) {
        constexpr int HH = decltype(tag)::H;
        if (plan)
            hipLaunchKernelGGL(softmax_segment_kernel<HH>, dim3(grid_for(plan->seg_capacity, 1, kPersistentBlocks)),
                               dim3(kBlock), 0, stream, scores, out, *plan);
        const int64_t waves = (n_rows + kSmRowsPerWave - 1) / kSmRowsPerWave;
        hipLaunchKernelGGL(softmax_short_kernel<HH>, dim3(grid_for(waves, kWavesPerBlock, INT32_MAX)), dim3(kBlock),
                           0, stream, row_ptr, n_rows, scores, out, plan ? plan->short_max : INT32_MAX);
        if (plan)
            hipLaunchKernelGGL(softmax_hub_write_kernel<HH>,
                               dim3(grid_for(plan->hubseg_capacity, 1, kPersistentBlocks)), dim3(kBlock), 0, stream,
                               row_ptr, scores, out, *plan);
    });
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gat
