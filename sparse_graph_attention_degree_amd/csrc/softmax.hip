// Row-wise multi-head edge softmax (POPCORNBENCH l1_p6, the reference model: for
// every node and head, softmax over the node's edge slice of scores [E,H],
// computed as exp(x - max) / sum(exp(x - max))).
//
// The page's kernels map one thread to a (node, head) pair striding through the
// slice with stride H, or one block per node with shared-memory reductions.
// Here, by degree:
//  * short rows (the common case): a wave takes 32 consecutive rows; their scores
//    form one contiguous run, which the wave stages into LDS with coalesced loads
//    (up to kBlkBudget floats at a time, whole rows).  One lane per (row, head)
//    then computes max, sum of exp and alpha from LDS, and the wave streams alpha
//    back with coalesced stores: one HBM round trip per group of rows.
//  * rows too long for the stage but not binned long (no plan, or a large
//    short_max): a 32-lane slot per row reads the row 32 values at a time (lane q:
//    edge q/H, head q%H), per-head max / sum are xor-shuffle trees over lanes q,
//    q^H, q^2H, ...; three passes: max, sum of exp, write.
//  * long rows and hub segments (the plan's segment table): a wave per segment,
//    streaming it in 1024-float chunks with a running (max, sum) per head; a row of
//    one chunk is written from registers.  Hub rows: their segments' (max, sum)
//    states merge, then a workgroup per segment writes alpha.
// Each (row, head) is reduced in an order fixed by the row alone, so a row's
// result does not depend on the rows around it (a batch of graphs gives every
// graph's rows the same bits as the graph alone).
#include <math.h>

#include "kernels.hpp"
#include "span.hpp"

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

constexpr int kBlkRows = 32;       // rows per wave (at most: fewer on graphs too small to fill the device)
constexpr int64_t kSmFillWaves = 2048;
constexpr int kBlkBudget = 1024;   // floats staged per wave (4 KB: 16 KB per workgroup, so LDS admits 10)

// Rows with 0 < deg <= hi (hi * H <= kBlkBudget): a wave per 32 consecutive rows, groups of
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
        // floats in the group, <= kBlkBudget (scalar: the buffer descriptors are built from it)
        const int len = __builtin_amdgcn_readfirstlane((last - base) * H);
        const int64_t run0 = (int64_t)__builtin_amdgcn_readfirstlane(base) * H;
        const __amdgpu_buffer_rsrc_t src = span(sc + run0, (int64_t)len * 4);
        const __amdgpu_buffer_rsrc_t dst = span(out + run0, (int64_t)len * 4);
        // stage the run (all loads issued before the first LDS write)
        float v[kBlkBudget / kWave];
        load_run(src, len, lane, v);
        wave_lds_handoff();   // the previous group's stage reads come before this rewrite
#pragma unroll
        for (int t = 0; t < kBlkBudget / kWave; ++t)
            if (t * kWave < len) stage[t * kWave + lane] = v[t];
        wave_lds_handoff();   // staged by lane l, read by the lane of each (row, head)
        // one lane per (row, head); the exponentials of the sum pass are kept in the stage and
        // scaled in place
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
                for (int x = b; x < e; ++x) {
                    const float ex = exp_fast(stage[x * H + h] - m);
                    stage[x * H + h] = ex;
                    z += ex;
                }
                const float rz = 1.f / z;
#pragma unroll 8
                for (int x = b; x < e; ++x) stage[x * H + h] *= rz;
            }
        }
        wave_lds_handoff();   // alpha written by the (row, head) lanes, stored by lane l
#pragma unroll
        for (int t = 0; t < kBlkBudget / kWave; ++t)
            if (t * kWave < len) bstore(dst, stage[t * kWave + lane], (lane + t * kWave) * 4);
        i = j;
    }
}

constexpr int kSegRegs = 16;                      // floats each lane holds of a segment chunk
constexpr int kWaveChunk = kSegRegs * kWave;       // 1024 floats per chunk

// One wave per plan segment (long rows, and hub segments whose (max, sum) states merge
// afterwards), with no barrier and no LDS, so every wave of the device streams a segment of its
// own.  A segment is read in chunks of kWaveChunk floats, kSegRegs per lane with coalesced
// loads: lane l holds elements l, l+64, ... of the chunk, all of head l % H (64 is a multiple of
// H, and every chunk starts on an edge and holds at least one element of every head).  Per chunk
// the head's maximum is an xor-shuffle tree over the head's lanes; each lane keeps a running sum
// of exp(s - max), rescaled when the maximum grows, and the sums of a head meet in a second
// tree at the end.  A segment of one chunk stays in registers from the read to the write; a
// longer long row is read again to write alpha.  Hub segments leave (max[H], sum[H]) in their
// partial slot.
template <int H>
__global__ __launch_bounds__(kBlock) void softmax_segment_kernel(const float* sc, float* out, PlanView plan) {
    const int lane = lane_id();
    const int64_t n_segs = plan.counts[kNSegs];
    const int64_t n_waves = (int64_t)gridDim.x * kWavesPerBlock;
    // the wave index as a scalar, so that the segment entry and the buffer descriptors built
    // from it stay in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    for (int64_t s = (int64_t)blockIdx.x * kWavesPerBlock + wave; s < n_segs; s += n_waves) {
        const int4 sg = plan.segs[s];
        const int64_t n = (int64_t)(sg.z - sg.y) * H;
        const float* seg = sc + (int64_t)sg.y * H;
        float v[kSegRegs];
        float m = -INFINITY, z = 0.f;
        for (int64_t c0 = 0; c0 < n; c0 += kWaveChunk) {
            const int cn = (int)(n - c0 < kWaveChunk ? n - c0 : kWaveChunk);
            const __amdgpu_buffer_rsrc_t src = span(seg + c0, (int64_t)cn * 4);
            load_run(src, cn, lane, v);
            float cm = -INFINITY;
#pragma unroll
            for (int k = 0; k < kSegRegs; ++k) {
                if (lane >= cn - k * kWave) v[k] = -INFINITY;   // scalar bound: no per-k lane index kept
                cm = fmaxf(cm, v[k]);
            }
#pragma unroll
            for (int o = H; o < kWave; o <<= 1) cm = fmaxf(cm, shfl_xor(cm, o));
            const float mn = fmaxf(m, cm);   // finite: the chunk holds an element of this head
            float cz = 0.f;
#pragma unroll
            for (int k = 0; k < kSegRegs; ++k)
                if (k * kWave < cn) cz += exp_fast(v[k] - mn);   // exp(-inf) = 0 past the end
            z = z * exp_fast(m - mn) + cz;                         // m = -inf on the first chunk: z = cz
            m = mn;
        }
#pragma unroll
        for (int o = H; o < kWave; o <<= 1) z += shfl_xor(z, o);
        if (sg.w >= 0) {
            if (lane < H) {
                float* prt = plan.partials + (int64_t)sg.w * plan.state_floats;
                prt[lane] = m;
                prt[H + lane] = z;
            }
            continue;
        }
        const float rz = 1.f / z;
        float* dseg = out + (int64_t)sg.y * H;
        if (n <= kWaveChunk) {
            const __amdgpu_buffer_rsrc_t dst = span(dseg, n * 4);
#pragma unroll
            for (int k = 0; k < kSegRegs; ++k)
                if (k * kWave < n) bstore(dst, exp_fast(v[k] - m) * rz, (lane + k * kWave) * 4);
            continue;
        }
        for (int64_t c0 = 0; c0 < n; c0 += kWaveChunk) {
            const int cn = (int)(n - c0 < kWaveChunk ? n - c0 : kWaveChunk);
            const __amdgpu_buffer_rsrc_t src = span(seg + c0, (int64_t)cn * 4);
            const __amdgpu_buffer_rsrc_t dst = span(dseg + c0, (int64_t)cn * 4);
            load_run(src, cn, lane, v);
#pragma unroll
            for (int k = 0; k < kSegRegs; ++k)
                if (k * kWave < cn) bstore(dst, exp_fast(v[k] - m) * rz, (lane + k * kWave) * 4);
        }
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

// One workgroup per hub segment: read the row's merged state, then write alpha.  The scores of
// a segment are read in batches, all loads of a batch issued before the first store (out may
// alias sc, so the compiler would otherwise keep each load-exp-store in order).  The batch loads
// do not depend on the merged state, so they are issued before it is fetched.  With H >= 4 and
// 16-byte aligned arrays a segment's run starts on a 16-byte boundary, and threads move 4
// consecutive floats at a time (heads (4t + j) % H, fixed per thread since 1024 is a multiple
// of H); otherwise one float at a time.
constexpr int kHubBatch = 16;   // floats per thread per batch

template <int H>
__global__ __launch_bounds__(kBlock) void softmax_hub_write_kernel(const int32_t* __restrict__ row_ptr,
                                                                   const float* sc, float* out, PlanView plan) {
    const int n_hub_segs = plan.counts[kNHubSegs];
    const bool wide = H >= 4 && ((reinterpret_cast<uintptr_t>(sc) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
    for (int s = blockIdx.x; s < n_hub_segs; s += gridDim.x) {
        const int4 sg = plan.segs[s];   // row, b, e, slot (= s)
        const int rb = row_ptr[sg.x];
        const int first = sg.w - (int)(((int64_t)sg.y - rb) / plan.seg_len);
        const float* p0 = plan.partials + (int64_t)first * plan.state_floats;
        const int64_t beg = (int64_t)sg.y * H, end = (int64_t)sg.z * H;
        if (wide) {
            constexpr int NB = kHubBatch / 4;   // float4 per thread per batch
            const float4* s4 = reinterpret_cast<const float4*>(sc + beg);
            float4* o4 = reinterpret_cast<float4*>(out + beg);
            const int64_t n4 = (end - beg) / 4;   // H >= 4: whole float4s
            for (int64_t f0 = threadIdx.x; f0 < n4; f0 += NB * kBlock) {
                float4 v[NB];
#pragma unroll
                for (int k = 0; k < NB; ++k) {
                    const int64_t f = f0 + (int64_t)k * kBlock;
                    v[k] = f < n4 ? s4[f] : make_float4(0.f, 0.f, 0.f, 0.f);
                }
                const int h0 = (4 * threadIdx.x) % H;
                float M[4], rz[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    M[j] = p0[(h0 + j) % H];
                    rz[j] = 1.f / p0[H + (h0 + j) % H];
                }
#pragma unroll
                for (int k = 0; k < NB; ++k) {
                    const int64_t f = f0 + (int64_t)k * kBlock;
                    if (f < n4)
                        o4[f] = make_float4(exp_fast(v[k].x - M[0]) * rz[0], exp_fast(v[k].y - M[1]) * rz[1],
                                            exp_fast(v[k].z - M[2]) * rz[2], exp_fast(v[k].w - M[3]) * rz[3]);
                }
            }
            continue;
        }
        // kBlock is a multiple of H, so every element this thread touches has head t % H
        const int h = threadIdx.x % H;
        for (int64_t i0 = beg + threadIdx.x; i0 < end; i0 += kHubBatch * kBlock) {
            float v[kHubBatch];
#pragma unroll
            for (int k = 0; k < kHubBatch; ++k) {
                const int64_t i = i0 + (int64_t)k * kBlock;
                v[k] = i < end ? sc[i] : 0.f;
            }
            const float M = p0[h], rz = 1.f / p0[H + h];
#pragma unroll
            for (int k = 0; k < kHubBatch; ++k) {
                const int64_t i = i0 + (int64_t)k * kBlock;
                if (i < end) out[i] = exp_fast(v[k] - M) * rz;
            }
        }
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
            hipLaunchKernelGGL(softmax_segment_kernel<HH>,
                               dim3(grid_for(plan->seg_capacity, kWavesPerBlock, kSegmentGrid)),
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
                               dim3(grid_for(plan->hubseg_capacity, 1, kSegmentGrid)), dim3(kBlock), 0, stream,
                               row_ptr, scores, out, *plan);
        }
    });
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gat
