// Row-wise multi-head edge softmax (POPCORNBENCH l1_p6, the reference model: for
// every node and head, softmax over the node's edge slice of scores [E,H],
// computed as exp(x - max) / sum(exp(x - max))).
//
// The page's kernels map one thread to a (node, head) pair striding through the
// slice with stride H, or one block per node with shared-memory reductions.
// Here, by degree:
//  * short rows (the common case): a wave takes 64 consecutive rows; their scores
//    form one contiguous run, which the wave stages into LDS with coalesced loads
//    (up to kBlkBudget floats at a time, whole rows).  One lane per (row, head)
//    then computes max, sum of exp and alpha from LDS, and the wave streams alpha
//    back with coalesced stores: one HBM round trip per group of rows.
//  * rows too long for the stage but not binned long (no plan, or a large
//    short_max): a 32-lane slot per row reads the row 32 values at a time (lane q:
//    edge q/H, head q%H), per-head max / sum are xor-shuffle trees over lanes q,
//    q^H, q^2H, ...; three passes: max, sum of exp, write.
//  * long rows: a workgroup per row, the row held in registers across the
//    workgroup (one coalesced read, one coalesced write); hub rows: segments across
//    workgroups whose (max, sum) states merge before alpha is written.
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

// one 32-lane slot per row, rows with lo < deg <= hi
template <int H>
__global__ __launch_bounds__(kBlock) void softmax_short_kernel(const int32_t* __restrict__ row_ptr, int64_t n_rows,
                                                               const float* sc, float* out, int lo, int hi) {
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
        if (!(wb + j < n_rows && e1 - e0 > lo && e1 - e0 <= hi)) e1 = e0;
        float m, z;
        sl.stats(sc, e0, e1, m, z);
        sl.write(sc, out, e0, e1, m, z);
    }
}

constexpr int kBlkRows = 64;       // rows per wave (at most: fewer on graphs too small to fill the device)
constexpr int64_t kSmFillWaves = 2048;
constexpr int kBlkBudget = 2048;   // floats staged per wave (8 KB)

// Rows with 0 < deg <= hi (hi * H <= kBlkBudget): a wave per 64 consecutive rows, groups of
// consecutive such rows staged in LDS.  A row of another class (non-empty, deg > hi) ends a
// group, since its scores sit between the groups' runs.
template <int H>
__global__ __launch_bounds__(kBlock) void softmax_block_kernel(const int32_t* __restrict__ row_ptr, int64_t n_rows,
                                                               const float* sc, float* out, int hi, int rpw) {
    __shared__ float stage_all[kWavesPerBlock][kBlkBudget];
    float* stage = stage_all[threadIdx.x / kWave];
    const int lane = lane_id();
    const int64_t r0 = ((int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave) * rpw;
    if (r0 >= n_rows) return;
    const int nr = (int)((n_rows - r0) < rpw ? (n_rows - r0) : rpw);
    int rb = 0, re = 0;
    if (lane < nr) {
        rb = row_ptr[r0 + lane];
        re = row_ptr[r0 + lane + 1];
    }
    const int deg = re - rb;
    const uint64_t mine = __ballot(lane < nr && deg > 0 && deg <= hi);
    const uint64_t breaker = __ballot(lane < nr && deg > hi);
    int i = 0;
    while (true) {
        // first row of the next group
        const uint64_t from_i = i < 64 ? (mine >> i) << i : 0ull;
        if (from_i == 0) break;
        i = __builtin_ctzll(from_i);
        // the group ends at the next breaker row or where the run would overflow the stage
        const uint64_t br = i < 63 ? (breaker >> (i + 1)) << (i + 1) : 0ull;
        const int jb = br ? __builtin_ctzll(br) : nr;
        const int base = shfl(rb, i);
        const uint64_t fits = __ballot(lane >= i && lane < jb && (int64_t)(re - base) * H <= kBlkBudget);
        const uint64_t nofit = ~fits & (jb < 64 ? (1ull << jb) - 1 : ~0ull) & ~((1ull << i) - 1);
        const int j = nofit ? __builtin_ctzll(nofit) : jb;
        const int last = shfl(re, j - 1);
        const int len = (last - base) * H;   // floats in the group, <= kBlkBudget
        const float* src = sc + (int64_t)base * H;
        float* dst = out + (int64_t)base * H;
        // stage the run (all loads issued before the first LDS write)
        float v[kBlkBudget / kWave];
#pragma unroll
        for (int t = 0; t < kBlkBudget / kWave; ++t)
            if (t * kWave < len && t * kWave + lane < len) v[t] = src[t * kWave + lane];
#pragma unroll
        for (int t = 0; t < kBlkBudget / kWave; ++t)
            if (t * kWave < len && t * kWave + lane < len) stage[t * kWave + lane] = v[t];
        // one lane per (row, head)
        const int pairs = (j - i) * H;
        for (int t = 0; t * kWave < pairs; ++t) {
            const int pp = t * kWave + lane;
            const bool live = pp < pairs;
            const int row = i + (live ? pp / H : 0);
            const int h = pp % H;
            const int b = shfl(rb, row) - base, e = shfl(re, row) - base;
            if (live) {
                float m = -INFINITY;
#pragma unroll 8
                for (int x = b; x < e; ++x) m = fmaxf(m, stage[x * H + h]);
                float z = 0.f;
#pragma unroll 8
                for (int x = b; x < e; ++x) z += exp_fast(stage[x * H + h] - m);
                const float rz = 1.f / z;
#pragma unroll 8
                for (int x = b; x < e; ++x) stage[x * H + h] = exp_fast(stage[x * H + h] - m) * rz;
            }
        }
#pragma unroll
        for (int t = 0; t < kBlkBudget / kWave; ++t)
            if (t * kWave < len && t * kWave + lane < len) dst[t * kWave + lane] = stage[t * kWave + lane];
        i = j;
    }
}

constexpr int kSegRegs = 32;                     // floats each thread holds of a segment
constexpr int kSegBudget = kSegRegs * kBlock;     // 8192: segments up to this many floats stay in registers

// One workgroup per plan segment.  A segment of up to kSegBudget floats is read once, with
// coalesced loads, into registers: thread t holds elements t, t+256, ... which all belong to
// head t % H (256 is a multiple of H), so per-head max and sum are a per-thread pass, an
// xor-shuffle tree over lanes of one head, and a 4-wave merge through LDS; alpha is then
// written from the registers.  Longer segments fall back to 8 slots (three passes each).
// Long rows are written here; hub segments leave (max[H], sum[H]) in the partial buffer.
template <int H>
__global__ __launch_bounds__(kBlock) void softmax_segment_kernel(const float* sc, float* out, PlanView plan) {
    constexpr int NS = kBlock / kSmG;
    __shared__ float lm[NS][H], lz[NS][H], gm[H], gz[H];
    const int lane = lane_id();
    const int t = threadIdx.x;
    const int w = t / kWave;
    const int gs = t / kSmG;
    SmSlot<H> sl;
    sl.q = lane % kSmG;
    const int n_segs = plan.counts[kNSegs];
    for (int s = blockIdx.x; s < n_segs; s += gridDim.x) {
        const int4 sg = plan.segs[s];
        const int64_t len = (int64_t)sg.z - sg.y;
        if (len * H <= kSegBudget) {
            const int n = (int)len * H;
            const int64_t off = (int64_t)sg.y * H;
            float v[kSegRegs];
            float m = -INFINITY;
#pragma unroll
            for (int k = 0; k < kSegRegs; ++k) {
                v[k] = -INFINITY;
                if (k * kBlock < n && t + k * kBlock < n) v[k] = sc[off + t + k * kBlock];
                m = fmaxf(m, v[k]);
            }
#pragma unroll
            for (int o = H; o < kWave; o <<= 1) m = fmaxf(m, shfl_xor(m, o));
            if (lane < H) lm[w][lane] = m;
            __syncthreads();
            const int h = t % H;
            float M = -INFINITY;
#pragma unroll
            for (int i = 0; i < kWavesPerBlock; ++i) M = fmaxf(M, lm[i][h]);
            float z = 0.f;
#pragma unroll
            for (int k = 0; k < kSegRegs; ++k)
                if (k * kBlock < n && t + k * kBlock < n) z += exp_fast(v[k] - M);
#pragma unroll
            for (int o = H; o < kWave; o <<= 1) z += shfl_xor(z, o);
            if (lane < H) lz[w][lane] = z;
            __syncthreads();
            float Z = 0.f;
#pragma unroll
            for (int i = 0; i < kWavesPerBlock; ++i) Z += lz[i][h];
            if (sg.w < 0) {
                const float rz = 1.f / Z;
#pragma unroll
                for (int k = 0; k < kSegRegs; ++k)
                    if (k * kBlock < n && t + k * kBlock < n) out[off + t + k * kBlock] = exp_fast(v[k] - M) * rz;
            } else if (t < H) {
                float* prt = plan.partials + (int64_t)sg.w * plan.state_floats;
                prt[t] = M;
                prt[H + t] = Z;
            }
            __syncthreads();
            continue;
        }
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

// One workgroup per hub row: merge its segments' (max, sum) states -- the 256 threads split
// the segments, then an xor-shuffle tree and a 4-wave merge -- and store the merged state in
// the slot of the row's first segment.
template <int H>
__global__ __launch_bounds__(kBlock) void softmax_hub_merge_kernel(PlanView plan) {
    __shared__ float lm[kWavesPerBlock][H], lz[kWavesPerBlock][H];
    const int t = threadIdx.x, lane = lane_id(), w = t / kWave;
    const int n_hubs = plan.counts[kNHubs];
    for (int hb = blockIdx.x; hb < n_hubs; hb += gridDim.x) {
        const int4 hr = plan.hubs[hb];   // row, first segment, n segments
        float* p0 = plan.partials + (int64_t)hr.y * plan.state_floats;
        float m[H], z[H];
#pragma unroll
        for (int h = 0; h < H; ++h) {
            m[h] = -INFINITY;
            z[h] = 0.f;
        }
        for (int c = t; c < hr.z; c += kBlock) {
            const float* pc = p0 + (int64_t)c * plan.state_floats;
#pragma unroll
            for (int h = 0; h < H; ++h) {
                const float mc = pc[h], zc = pc[H + h];
                const float mn = fmaxf(m[h], mc);
                z[h] = (m[h] == -INFINITY ? 0.f : z[h] * exp_fast(m[h] - mn)) +
                       (mc == -INFINITY ? 0.f : zc * exp_fast(mc - mn));
                m[h] = mn;
            }
        }
#pragma unroll
        for (int h = 0; h < H; ++h) {
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const float mo = shfl_xor(m[h], o), zo = shfl_xor(z[h], o);
                const float mn = fmaxf(m[h], mo);
                z[h] = (m[h] == -INFINITY ? 0.f : z[h] * exp_fast(m[h] - mn)) +
                       (mo == -INFINITY ? 0.f : zo * exp_fast(mo - mn));
                m[h] = mn;
            }
            if (lane == 0) {
                lm[w][h] = m[h];
                lz[w][h] = z[h];
            }
        }
        __syncthreads();
        if (t < H) {
            float M = -INFINITY, Z = 0.f;
#pragma unroll
            for (int i = 0; i < kWavesPerBlock; ++i) M = fmaxf(M, lm[i][t]);
#pragma unroll
            for (int i = 0; i < kWavesPerBlock; ++i)
                if (lm[i][t] != -INFINITY) Z = fmaf(lz[i][t], exp_fast(lm[i][t] - M), Z);
            p0[t] = M;
            p0[H + t] = Z;
        }
        __syncthreads();
    }
}

// One workgroup per hub segment: read the row's merged state, then write alpha.
template <int H>
__global__ __launch_bounds__(kBlock) void softmax_hub_write_kernel(const int32_t* __restrict__ row_ptr,
                                                                   const float* sc, float* out, PlanView plan) {
    const int n_hub_segs = plan.counts[kNHubSegs];
    for (int s = blockIdx.x; s < n_hub_segs; s += gridDim.x) {
        const int4 sg = plan.segs[s];   // row, b, e, slot (= s)
        const int rb = row_ptr[sg.x];
        const int first = sg.w - (int)(((int64_t)sg.y - rb) / plan.seg_len);
        const float* p0 = plan.partials + (int64_t)first * plan.state_floats;
        // kBlock is a multiple of H, so every element this thread touches has head t % H
        const int h = threadIdx.x % H;
        const float M = p0[h], rz = 1.f / p0[H + h];
        for (int64_t i = (int64_t)sg.y * H + threadIdx.x; i < (int64_t)sg.z * H; i += kBlock)
            out[i] = exp_fast(sc[i] - M) * rz;
    }
}

}  // namespace

hipError_t launch_softmax(int H, const int32_t* row_ptr, int64_t n_rows, const float* scores, float* out,
                          const PlanView* plan, hipStream_t stream) {
    const bool ok = dispatch_heads(H, [&](auto tag) {
        constexpr int HH = decltype(tag)::H;
        const int short_max = plan ? plan->short_max : INT32_MAX;
        const int staged = short_max < kBlkBudget / HH ? short_max : kBlkBudget / HH;   // rows the stage takes
        if (plan)
            hipLaunchKernelGGL(softmax_segment_kernel<HH>, dim3(grid_for(plan->seg_capacity, 1, kPersistentBlocks)),
                               dim3(kBlock), 0, stream, scores, out, *plan);
        int64_t rpw = (n_rows + kSmFillWaves - 1) / kSmFillWaves;   // enough waves to fill the device
        rpw = rpw < 1 ? 1 : (rpw > kBlkRows ? kBlkRows : rpw);
        const int64_t bwaves = (n_rows + rpw - 1) / rpw;
        hipLaunchKernelGGL(softmax_block_kernel<HH>, dim3(grid_for(bwaves, kWavesPerBlock, INT32_MAX)), dim3(kBlock),
                           0, stream, row_ptr, n_rows, scores, out, staged, (int)rpw);
        if (short_max > staged) {
            const int64_t waves = (n_rows + kSmRowsPerWave - 1) / kSmRowsPerWave;
            hipLaunchKernelGGL(softmax_short_kernel<HH>, dim3(grid_for(waves, kWavesPerBlock, INT32_MAX)),
                               dim3(kBlock), 0, stream, row_ptr, n_rows, scores, out, staged, short_max);
        }
        if (plan) {
            hipLaunchKernelGGL(softmax_hub_merge_kernel<HH>, dim3(grid_for(plan->hub_capacity, 1, kPersistentBlocks)),
                               dim3(kBlock), 0, stream, *plan);
            hipLaunchKernelGGL(softmax_hub_write_kernel<HH>,
                               dim3(grid_for(plan->hubseg_capacity, 1, kPersistentBlocks)), dim3(kBlock), 0, stream,
                               row_ptr, scores, out, *plan);
        }
    });
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gat
