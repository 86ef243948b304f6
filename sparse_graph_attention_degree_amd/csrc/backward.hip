// Backward of the path, and the transposed (CSC) view of the graph that it needs.
//
// The forward steps are out[i] = sum over row i of w[e] * x[col[e]] and its softmax / SDDMM
// relatives.  Their gradients with respect to the gathered tables sum over the edges that read
// each source row.  The SDDMM page (POPCORNBENCH l1_p10, the passage on the backward pass) has
// those sums done with atomic additions; here they are plain gathers over the transposed graph
// (sources as rows), built once per graph by a stable sort of the edges by column, so the
// transposed aggregation reuses the forward kernels and every sum has a fixed order.
//
// Kernels in this file:
//  * expand_rows: row id of every CSR edge.
//  * radix_hist / radix_scatter: one pass of an LSD radix sort (digits of up to 8 bits) of
//    (column, edge id) pairs, stable, so the final order is by column and then by edge id; scan_*:
//    the exclusive scan of the per-tile digit counts between the two.
//  * csc_bounds: column pointers from the sorted columns (the row of each CSC entry rides along
//    through the sort as a second value).
//  * permute_edges: per-edge values [E,H] moved into CSC order.
//  * edge_dot: per edge and head, <G[row(e)], F[col(e)]> with G fp32 and F fp32 or bf16 (the
//    gradient of the aggregation weights, and of the softmax output in the fused backward).
//  * softmax_bwd_*: out = scale * alpha * (g - sum_row alpha * g), by degree class like the
//    forward.
#include <math.h>

#include "kernels.hpp"
#include "span.hpp"

namespace gat {

namespace {

// ------------------------------------------------------------------------------ row ids
// A wave per 64 rows: a row of up to 64 edges is written by its own lane, a longer one by the
// whole wave.
__global__ __launch_bounds__(kBlock) void expand_rows_kernel(const int32_t* __restrict__ row_ptr, int64_t n_rows,
                                                             int32_t* __restrict__ rows) {
    const int lane = lane_id();
    const int64_t r0 = ((int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave) * kWave;
    if (r0 >= n_rows) return;
    const int64_t r = r0 + lane;
    int b = 0, e = 0;
    if (r < n_rows) {
        b = row_ptr[r];
        e = row_ptr[r + 1];
    }
    if (e - b <= kWave)
        for (int x = b; x < e; ++x) rows[x] = (int32_t)r;
    uint64_t big = __ballot(r < n_rows && e - b > kWave);
    while (big) {
        const int l = __builtin_ctzll(big);
        big &= big - 1;
        const int bb = shfl(b, l), ee = shfl(e, l);
        for (int x = bb + lane; x < ee; x += kWave) rows[x] = (int32_t)(r0 + l);
    }
}

// ------------------------------------------------------------------------------ radix sort
// One LSD pass on a digit of `bits` <= 8 bits.  A tile is 4096 consecutive items, 1024 per wave in
// 16 rounds of 64 (round k, lane l: item k*64 + l of the wave's run).  In each round the lanes
// holding the same digit find each other with one ballot per digit bit; a lane's stable rank in the
// wave is the wave's running count of its digit (LDS) plus the same-digit lanes below it.  After
// the rounds the per-wave counts give each digit's start in the tile, the items are placed in LDS in
// (digit, rank) order, and the tile is written out in that order: consecutive threads write
// consecutive positions of one digit's run, so the stores are coalesced runs instead of one scattered
// 4-byte store per item.
constexpr int kSortItems = 16;
constexpr int kSortTile = kBlock * kSortItems;
constexpr int kWaveRun = kSortTile / kWavesPerBlock;

__global__ __launch_bounds__(kBlock) void radix_hist_kernel(const int32_t* __restrict__ keys, int64_t n, int shift,
                                                            int bits, int32_t* __restrict__ hist, int64_t n_tiles) {
    __shared__ int cnt[kRadixMaxBins];
    const int t = threadIdx.x;
    const int bins = 1 << bits, mask = bins - 1;
    cnt[t] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kSortTile;
#pragma unroll
    for (int k = 0; k < kSortItems; ++k) {
        const int64_t i = base + (int64_t)k * kBlock + t;
        if (i < n) atomicAdd(&cnt[(keys[i] >> shift) & mask], 1);
    }
    __syncthreads();
    if (t < bins) hist[(int64_t)t * n_tiles + blockIdx.x] = cnt[t];
}

__device__ int block_exscan_int(int v, int& total);

// vin == nullptr: the values are the item positions (the first pass, identity order).
// offs[d * n_tiles + tile]: the output position of the tile's first item of digit d.
// V2: a second value per item (v2in -> v2out) moves with the key, so that a payload known in the
// input order (the row of a CSR edge, the other end of a COO edge) arrives sorted without a gather
// through the permutation afterwards.
template <bool V2>
__global__ __launch_bounds__(kBlock) void radix_scatter_kernel(const int32_t* __restrict__ kin,
                                                               const int32_t* __restrict__ vin,
                                                               int32_t* __restrict__ kout, int32_t* __restrict__ vout,
                                                               const int32_t* __restrict__ v2in,
                                                               int32_t* __restrict__ v2out, int64_t n, int shift,
                                                               int bits, const int32_t* __restrict__ offs,
                                                               int64_t n_tiles) {
    __shared__ int wcnt[kWavesPerBlock][kRadixMaxBins];   // per wave and digit: count, then the wave's base
    __shared__ int dstart[kRadixMaxBins];                   // digit's first slot in the tile
    __shared__ int dglobal[kRadixMaxBins];                  // output position of slot 0 of the digit's run
    __shared__ int skey[kSortTile], sval[kSortTile];
    __shared__ int sval2[V2 ? kSortTile : 1];
    const int t = threadIdx.x, lane = lane_id(), w = t / kWave;
    const int bins = 1 << bits, mask = bins - 1;
    const int64_t tile0 = (int64_t)blockIdx.x * kSortTile;
    const int64_t run0 = tile0 + (int64_t)w * kWaveRun;
    const uint64_t below_me = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
    for (int wv = 0; wv < kWavesPerBlock; ++wv) wcnt[wv][t] = 0;
    __syncthreads();
    int key[kSortItems], val[kSortItems], rank[kSortItems], val2[V2 ? kSortItems : 1];
#pragma unroll
    for (int k = 0; k < kSortItems; ++k) {
        const int64_t i = run0 + (int64_t)k * kWave + lane;
        const bool valid = i < n;
        key[k] = valid ? kin[i] : 0;
        val[k] = valid ? (vin ? vin[i] : (int32_t)i) : 0;
        if constexpr (V2) val2[k] = valid ? v2in[i] : 0;
    }
#pragma unroll
    for (int k = 0; k < kSortItems; ++k) {
        const bool valid = run0 + (int64_t)k * kWave + lane < n;
        const int d = (key[k] >> shift) & mask;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < bits; ++b) {
            const uint64_t set = __ballot((d >> b) & 1);
            peers &= ((d >> b) & 1) ? set : ~set;
        }
        const int below = __popcll(peers & below_me);
        const int before = wcnt[w][d];
        rank[k] = before + below;
        wave_lds_handoff();   // every lane has read the counts before the run's first lane bumps them
        if (valid && below == 0) wcnt[w][d] = before + __popcll(peers);
        wave_lds_handoff();
    }
    __syncthreads();
    // digit t: the waves' bases within the digit (in wave order), then the digit's start in the tile
    int tot = 0;
    if (t < bins) {
#pragma unroll
        for (int wv = 0; wv < kWavesPerBlock; ++wv) {
            const int c = wcnt[wv][t];
            wcnt[wv][t] = tot;
            tot += c;
        }
    }
    int all;
    const int ex = block_exscan_int(t < bins ? tot : 0, all);
    if (t < bins) {
        dstart[t] = ex;
        dglobal[t] = offs[(int64_t)t * n_tiles + blockIdx.x] - ex;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kSortItems; ++k) {
        if (run0 + (int64_t)k * kWave + lane < n) {
            const int d = (key[k] >> shift) & mask;
            const int slot = dstart[d] + wcnt[w][d] + rank[k];
            skey[slot] = key[k];
            sval[slot] = val[k];
            if constexpr (V2) sval2[slot] = val2[k];
        }
    }
    __syncthreads();
    const int tile_n = (int)(n - tile0 < kSortTile ? n - tile0 : kSortTile);
    for (int i = t; i < tile_n; i += kBlock) {
        const int kk = skey[i];
        const int64_t pos = (int64_t)dglobal[(kk >> shift) & mask] + i;
        kout[pos] = kk;
        vout[pos] = sval[i];
        if constexpr (V2) v2out[pos] = sval2[i];
    }
}

// ------------------------------------------------------------------------------ exclusive scan
// out[i] = sum of in[0..i) for n int32 values (totals below 2^31); out may alias in.
constexpr int kScanItems = 16;
constexpr int kScanTile = kBlock * kScanItems;

__device__ int block_exscan_int(int v, int& total) {
    __shared__ int wsum[kWavesPerBlock];
    const int lane = lane_id(), w = threadIdx.x / kWave;
    int inc = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int u = __shfl_up(inc, o);
        if (lane >= o) inc += u;
    }
    if (lane == kWave - 1) wsum[w] = inc;
    __syncthreads();
    int off = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < kWavesPerBlock; ++i) {
        if (i < w) off += wsum[i];
        total += wsum[i];
    }
    __syncthreads();
    return off + inc - v;
}

__global__ __launch_bounds__(kBlock) void scan_reduce_kernel(const int32_t* __restrict__ in, int64_t n,
                                                             int32_t* __restrict__ sums) {
    const int64_t i0 = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanItems;
    int s = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k)
        if (i0 + k < n) s += in[i0 + k];
    int total;
    block_exscan_int(s, total);
    if (threadIdx.x == 0) sums[blockIdx.x] = total;
}

// one workgroup: exclusive scan of the tile sums, in place
__global__ __launch_bounds__(kBlock) void scan_sums_kernel(int32_t* __restrict__ sums, int64_t n) {
    int carry = 0;
    for (int64_t base = 0; base < n; base += kBlock) {
        const int64_t i = base + threadIdx.x;
        const int v = i < n ? sums[i] : 0;
        int total;
        const int ex = block_exscan_int(v, total);
        if (i < n) sums[i] = carry + ex;
        carry += total;
    }
}

__global__ __launch_bounds__(kBlock) void scan_apply_kernel(const int32_t* in, int64_t n,
                                                            const int32_t* __restrict__ sums, int32_t* out) {
    const int64_t i0 = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanItems;
    int v[kScanItems];
    int s = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        v[k] = i0 + k < n ? in[i0 + k] : 0;
        s += v[k];
    }
    int total;
    int run = sums[blockIdx.x] + block_exscan_int(s, total);
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        if (i0 + k < n) out[i0 + k] = run;
        run += v[k];
    }
}

// ------------------------------------------------------------------------------ CSC assembly
// Entry p of the sorted columns starts columns (previous column, column at p]: they all begin at p.
// p = n_edges closes the remaining columns up to n_src.
__global__ __launch_bounds__(kBlock) void csc_bounds_kernel(const int32_t* __restrict__ skeys, int64_t n_edges,
                                                            int64_t n_src, int32_t* __restrict__ col_ptr) {
    for (int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x; p <= n_edges; p += (int64_t)gridDim.x * kBlock) {
        const int64_t prev = p > 0 ? skeys[p - 1] : -1;
        const int64_t cur = p < n_edges ? skeys[p] : n_src;
        for (int64_t j = prev + 1; j <= cur; ++j) col_ptr[j] = (int32_t)p;
    }
}

// dst[p,:] = scale * src[perm[p],:] for [E,H] per-edge values (scale 1 moves the bits unchanged)
template <int H>
__global__ __launch_bounds__(kBlock) void permute_edges_kernel(const int32_t* __restrict__ perm,
                                                               const float* __restrict__ src, int64_t n,
                                                               float scale, float* __restrict__ dst) {
    for (int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x; p < n; p += (int64_t)gridDim.x * kBlock) {
        const int64_t e = perm[p];
        if constexpr (H % 4 == 0) {
#pragma unroll
            for (int h = 0; h < H; h += 4) {
                float4 x = *reinterpret_cast<const float4*>(src + e * H + h);
                x.x *= scale;
                x.y *= scale;
                x.z *= scale;
                x.w *= scale;
                *reinterpret_cast<float4*>(dst + p * H + h) = x;
            }
        } else {
#pragma unroll
            for (int h = 0; h < H; ++h) dst[p * H + h] = scale * src[e * H + h];
        }
    }
}

// ------------------------------------------------------------------------------ edge dots
// Per edge e (row i = rows[e], source j = col[e]) and head h: out[e,h] = <G[i,h,:], F[j,h,:]>,
// G fp32.  A slot of lanes holds one edge (the geometry of F's rows); each lane reads NV 16-byte
// pieces of F and the matching EPP floats of G; the head sums stay in registers (group_sum).

template <typename T, int H, int D>
__global__ __launch_bounds__(kBlock) void edge_dot_kernel(const int32_t* __restrict__ rows,
                                                          const int32_t* __restrict__ col, int64_t n_edges,
                                                          const float* __restrict__ gf, const T* __restrict__ ff,
                                                          float* __restrict__ out) {
    using Gm = Geo<T, H, D>;
    constexpr int G = Gm::G, P = Gm::P, NV = Gm::NV, EPP = Gm::EPP, LPH = Gm::LPH, HD = Gm::HD;
    constexpr int UMAX = (8 / NV) > 1 ? (8 / NV) : 1;   // up to 8 pieces of each row in flight per lane
    constexpr int U = UMAX * P <= kWave ? UMAX : kWave / P;
    constexpr int EPI = U * P;   // edges per wave iteration (<= 64: one index per lane)
    const int lane = lane_id();
    const int q = lane % G, g = lane / G;
    int hv[NV], off[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        hv[v] = (v * G + q) / LPH;
        off[v] = (v * G + q) * EPP;
    }
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t base = ((int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave) * EPI; base < n_edges;
         base += nwaves * EPI) {
        int ri = 0, ci = 0;
        if (lane < EPI && base + lane < n_edges) {
            ri = rows[base + lane];
            ci = col[base + lane];
        }
        uint4 fa[U][NV];
        float4 ga[U][NV][EPP / 4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int el = u * P + g;
            const int r_i = shfl(ri, el), c_i = shfl(ci, el);
            const bool valid = base + el < n_edges;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                if (valid) {
                    fa[u][v] = ld16(ff + (int64_t)c_i * HD + off[v]);
#pragma unroll
                    for (int k = 0; k < EPP / 4; ++k)
                        ga[u][v][k] = *reinterpret_cast<const float4*>(gf + (int64_t)r_i * HD + off[v] + 4 * k);
                } else {
                    fa[u][v] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
                    for (int k = 0; k < EPP / 4; ++k) ga[u][v][k] = make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int el = u * P + g;
            const int64_t e = base + el;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                float f[EPP];
                unpack<T>(fa[u][v], f);
                float d = 0.f;
#pragma unroll
                for (int k = 0; k < EPP / 4; ++k) {
                    d = fmaf(ga[u][v][k].x, f[4 * k], d);
                    d = fmaf(ga[u][v][k].y, f[4 * k + 1], d);
                    d = fmaf(ga[u][v][k].z, f[4 * k + 2], d);
                    d = fmaf(ga[u][v][k].w, f[4 * k + 3], d);
                }
                d = group_sum<LPH>(d);
                if (e < n_edges && (v * G + q) % LPH == 0) out[e * H + hv[v]] = d;
            }
        }
    }
}

// ------------------------------------------------------------------------------ softmax backward
// out[e,h] = scale * alpha[e,h] * (g[e,h] - sum_{e' in row} alpha[e',h] * g[e',h]); out may alias g.
constexpr int kSbG = 32;                  // lanes per row slot: lane q reads edge q/H, head q%H
constexpr int kSbRowsPerWave = 32;        // at most; a multiple of the 2 slots per wave
constexpr int64_t kSbFillWaves = 2048;
constexpr int kSbRegs = 8;                // rows of up to 8 values per lane are held in registers

// rows with deg <= hi (all rows when there is no plan), a 32-lane slot per row: one pass for the
// per-head dot, one for the output
template <int H>
__global__ __launch_bounds__(kBlock) void softmax_bwd_short_kernel(const int32_t* __restrict__ row_ptr,
                                                                   int64_t n_rows, const float* alpha,
                                                                   const float* grad, float* out, int hi,
                                                                   float scale, int rpw) {
    constexpr int SC = kSbG / H;
    const int lane = lane_id();
    const int64_t wb = ((int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave) * rpw;
    if (wb >= n_rows) return;
    int rpv = 0;
    if (lane <= rpw && wb + lane <= n_rows) rpv = row_ptr[wb + lane];
    const int q = lane % kSbG, g = lane / kSbG, es = q / H;
#pragma unroll 1
    for (int it = 0; it < rpw / (kWave / kSbG); ++it) {
        const int j = it * (kWave / kSbG) + g;
        int e0 = shfl(rpv, j), e1 = shfl(rpv, j + 1);
        if (!(wb + j < n_rows && e1 - e0 <= hi)) e1 = e0;
        if (e1 - e0 <= kSbRegs * SC) {
            // the row in registers: lane q holds elements q, q+32, ... of its run; all loads are
            // issued before the first use
            const int n = (e1 - e0) * H;
            const int64_t r0 = (int64_t)e0 * H + q;
            float a[kSbRegs], gr[kSbRegs];
#pragma unroll
            for (int k = 0; k < kSbRegs; ++k) {
                const bool live = q + k * kSbG < n;
                a[k] = live ? alpha[r0 + k * kSbG] : 0.f;
                gr[k] = live ? grad[r0 + k * kSbG] : 0.f;
            }
            float s = 0.f;
#pragma unroll
            for (int k = 0; k < kSbRegs; ++k) s = fmaf(a[k], gr[k], s);
#pragma unroll
            for (int o = H; o < kSbG; o <<= 1) s += shfl_xor(s, o);
#pragma unroll
            for (int k = 0; k < kSbRegs; ++k)
                if (q + k * kSbG < n) out[r0 + k * kSbG] = scale * a[k] * (gr[k] - s);
            continue;
        }
        float s = 0.f;
        for (int c = e0; c < e1; c += SC)
            if (c + es < e1) {
                const int64_t i = (int64_t)c * H + q;
                s = fmaf(alpha[i], grad[i], s);
            }
#pragma unroll
        for (int o = H; o < kSbG; o <<= 1) s += shfl_xor(s, o);
        for (int c = e0; c < e1; c += SC)
            if (c + es < e1) {
                const int64_t i = (int64_t)c * H + q;
                out[i] = scale * alpha[i] * (grad[i] - s);
            }
    }
}

// workgroup-wide per-head sum of one float per thread, where thread t holds head t % H
template <int H>
__device__ __forceinline__ float block_head_sum(float s, float (*ls)[H]) {
    const int lane = lane_id(), w = threadIdx.x / kWave;
#pragma unroll
    for (int o = H; o < kWave; o <<= 1) s += shfl_xor(s, o);
    if (lane < H) ls[w][lane] = s;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < kWavesPerBlock; ++i) t += ls[i][threadIdx.x % H];
    __syncthreads();
    return t;
}

// One wave per plan segment, no barrier: the segment streams through in 1024-float chunks of
// alpha and grad (lane l holds elements l, l+64, ..., all of head l % H), the per-head dot is a
// per-lane sum and an xor-shuffle tree over the head's lanes; a one-chunk long row is written from
// registers, a longer one is read again; a hub segment leaves its per-head dot in the partial
// buffer.  One register set per lane holds alpha and grad of one chunk.  Left to itself the
// compiler keeps the first pass's registers apart from the write pass's and takes about 108
// VGPRs (4 waves per SIMD); asking for 6 waves per SIMD packs it into 80 without spilling.
constexpr int kSbSegRegs = 16;
constexpr int kSbChunk = kSbSegRegs * kWave;

template <int H>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(6))) void softmax_bwd_segment_kernel(const float* alpha, const float* grad,
                                                                     float* out, PlanView plan, float scale) {
    const int lane = lane_id();
    const int64_t n_segs = plan.counts[kNSegs];
    const int64_t n_waves = (int64_t)gridDim.x * kWavesPerBlock;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);   // scalar: see span.hpp
#pragma unroll 1
    for (int64_t s = (int64_t)blockIdx.x * kWavesPerBlock + wave; s < n_segs; s += n_waves) {
        const int4 sg = plan.segs[s];
        const int64_t n = (int64_t)(sg.z - sg.y) * H;
        const int64_t off = (int64_t)sg.y * H;
        // floats of the chunk at c0, 0 past the end (its loads then read 0 and move no data)
        auto chunk_len = [&](int64_t c0) {
            return opaque_uniform((int)(n - c0 <= 0 ? 0 : (n - c0 < kSbChunk ? n - c0 : kSbChunk)));
        };
        // a chunk of alpha and grad, every load issued (past the end: 0), so the compiler counts
        // them exactly and a wait for one chunk never covers the next one's loads
        auto load_chunk = [&](float(&x)[kSbSegRegs], float(&y)[kSbSegRegs], int64_t c0, int cn) {
            const __amdgpu_buffer_rsrc_t ra = span(alpha + off + c0, (int64_t)cn * 4);
            const __amdgpu_buffer_rsrc_t rg = span(grad + off + c0, (int64_t)cn * 4);
            const int b = opaque(lane * 4);
#pragma unroll
            for (int k = 0; k < kSbSegRegs; ++k) x[k] = bload(ra, b + k * kWave * 4);
#pragma unroll
            for (int k = 0; k < kSbSegRegs; ++k) y[k] = bload(rg, b + k * kWave * 4);
        };
        auto dot_chunk = [&](const float(&x)[kSbSegRegs], const float(&y)[kSbSegRegs], float& d) {
#pragma unroll
            for (int k = 0; k < kSbSegRegs; ++k) d = fmaf(x[k], y[k], d);   // 0 past the end
        };
        auto store_chunk = [&](const float(&x)[kSbSegRegs], const float(&y)[kSbSegRegs], int64_t c0, int cn,
                               float d) {
            const __amdgpu_buffer_rsrc_t dst = span(out + off + c0, (int64_t)cn * 4);
            const int b = opaque(lane * 4);
#pragma unroll
            for (int k = 0; k < kSbSegRegs; ++k) bstore(dst, scale * x[k] * (y[k] - d), b + k * kWave * 4);
        };
        float a[kSbSegRegs], g[kSbSegRegs];
        float dot = 0.f;
        int cv = 0;
#pragma unroll 1
        for (int64_t c0 = 0; c0 < n; c0 += kSbChunk) {
            cv = chunk_len(c0);
            load_chunk(a, g, c0, cv);
            dot_chunk(a, g, dot);
        }
#pragma unroll
        for (int o = H; o < kWave; o <<= 1) dot += shfl_xor(dot, o);
        if (sg.w >= 0) {
            if (lane < H) plan.partials[(int64_t)sg.w * plan.state_floats + lane] = dot;
            continue;
        }
        if (n <= kSbChunk) {
            // still in registers; only the stores that hold data are issued
            const __amdgpu_buffer_rsrc_t dst = span(out + off, (int64_t)cv * 4);
            const int b = opaque(lane * 4);
#pragma unroll
            for (int k = 0; k < kSbSegRegs; ++k)
                if (k * kWave < cv) bstore(dst, scale * a[k] * (g[k] - dot), b + k * kWave * 4);
            continue;
        }
#pragma unroll 1
        for (int64_t c0 = 0; c0 < n; c0 += kSbChunk) {
            cv = chunk_len(c0);
            load_chunk(a, g, c0, cv);
            store_chunk(a, g, c0, cv, dot);
        }
    }
}

// one workgroup per hub segment: the hub's dot is the sum of its segments' partials
constexpr int kSbHubBatch = 8;

template <int H>
__global__ __launch_bounds__(kBlock) void softmax_bwd_hub_kernel(const int32_t* __restrict__ row_ptr,
                                                                 const float* alpha, const float* grad, float* out,
                                                                 PlanView plan, float scale) {
    __shared__ float ls[kWavesPerBlock][H];
    const int t = threadIdx.x;
    const int n_hub_segs = plan.counts[kNHubSegs];
    for (int s = blockIdx.x; s < n_hub_segs; s += gridDim.x) {
        const int4 sg = plan.segs[s];   // row, b, e, slot (= s)
        const int rb = row_ptr[sg.x], re = row_ptr[sg.x + 1];
        const int first = sg.w - (int)(((int64_t)sg.y - rb) / plan.seg_len);
        const int nseg = (int)(((int64_t)re - rb + plan.seg_len - 1) / plan.seg_len);
        // kBlock is a multiple of H: thread t sums head t % H over segments t / H, t / H + 256 / H, ...
        float acc = 0.f;
        for (int c = t / H; c < nseg; c += kBlock / H)
            acc += plan.partials[(int64_t)(first + c) * plan.state_floats + t % H];
        const float dot = block_head_sum<H>(acc, ls);
        // batches of kSbHubBatch elements per thread, all loads before the first store (out may
        // alias grad)
        const int64_t end = (int64_t)sg.z * H;
        for (int64_t i0 = (int64_t)sg.y * H + t; i0 < end; i0 += kSbHubBatch * kBlock) {
            float a[kSbHubBatch], g[kSbHubBatch];
#pragma unroll
            for (int k = 0; k < kSbHubBatch; ++k) {
                const int64_t i = i0 + (int64_t)k * kBlock;
                a[k] = i < end ? alpha[i] : 0.f;
                g[k] = i < end ? grad[i] : 0.f;
            }
#pragma unroll
            for (int k = 0; k < kSbHubBatch; ++k) {
                const int64_t i = i0 + (int64_t)k * kBlock;
                if (i < end) out[i] = scale * a[k] * (g[k] - dot);
            }
        }
    }
}

}  // namespace

// ------------------------------------------------------------------------------ launchers
hipError_t launch_expand_rows(const int32_t* row_ptr, int64_t n_rows, int32_t* rows, hipStream_t stream) {
    if (n_rows == 0) return hipSuccess;
    const int64_t waves = (n_rows + kWave - 1) / kWave;
    hipLaunchKernelGGL(expand_rows_kernel, dim3(grid_for(waves, kWavesPerBlock, INT32_MAX)), dim3(kBlock), 0, stream,
                       row_ptr, n_rows, rows);
    return hipGetLastError();
}

int64_t radix_tiles(int64_t n) { return (n + kSortTile - 1) / kSortTile; }
int64_t scan_tiles(int64_t n) { return (n + kScanTile - 1) / kScanTile; }

hipError_t launch_exclusive_scan(const int32_t* in, int64_t n, int32_t* sums, int32_t* out, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const int64_t nb = scan_tiles(n);
    hipLaunchKernelGGL(scan_reduce_kernel, dim3((unsigned)nb), dim3(kBlock), 0, stream, in, n, sums);
    hipLaunchKernelGGL(scan_sums_kernel, dim3(1), dim3(kBlock), 0, stream, sums, nb);
    hipLaunchKernelGGL(scan_apply_kernel, dim3((unsigned)nb), dim3(kBlock), 0, stream, in, n, sums, out);
    return hipGetLastError();
}

hipError_t launch_radix_pass(const int32_t* kin, const int32_t* vin, int32_t* kout, int32_t* vout,
                             const int32_t* v2in, int32_t* v2out, int64_t n, int shift, int bits, int32_t* hist,
                             int32_t* sums, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    if (bits < 1 || bits > kRadixMaxBits || shift < 0 || shift > 30) return hipErrorInvalidValue;
    if ((v2in == nullptr) != (v2out == nullptr)) return hipErrorInvalidValue;
    const int64_t nt = radix_tiles(n);
    hipLaunchKernelGGL(radix_hist_kernel, dim3((unsigned)nt), dim3(kBlock), 0, stream, kin, n, shift, bits, hist, nt);
    const hipError_t e = launch_exclusive_scan(hist, nt << bits, sums, hist, stream);
    if (e != hipSuccess) return e;
    if (v2out)
        hipLaunchKernelGGL(radix_scatter_kernel<true>, dim3((unsigned)nt), dim3(kBlock), 0, stream, kin, vin, kout,
                           vout, v2in, v2out, n, shift, bits, hist, nt);
    else
        hipLaunchKernelGGL(radix_scatter_kernel<false>, dim3((unsigned)nt), dim3(kBlock), 0, stream, kin, vin, kout,
                           vout, v2in, v2out, n, shift, bits, hist, nt);
    return hipGetLastError();
}

RadixPlan radix_plan(int64_t n_keys) {
    int bits = 0;
    while (bits < 31 && ((int64_t)1 << bits) < n_keys) ++bits;   // keys are < n_keys
    RadixPlan p;
    p.passes = bits == 0 ? 1 : (bits + kRadixMaxBits - 1) / kRadixMaxBits;
    p.bits = bits == 0 ? 1 : (bits + p.passes - 1) / p.passes;
    return p;
}

hipError_t launch_bounds_from_keys(const int32_t* skeys, int64_t n_edges, int64_t n_rows, int32_t* row_ptr,
                                   hipStream_t stream) {
    hipLaunchKernelGGL(csc_bounds_kernel, dim3(grid_for(n_edges + 1, kBlock, 65536)), dim3(kBlock), 0, stream, skeys,
                       n_edges, n_rows, row_ptr);
    return hipGetLastError();
}

hipError_t launch_permute_edges(int H, const int32_t* perm, const float* src, int64_t n, float scale, float* dst,
                                hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const bool ok = dispatch_heads(H, [&](auto tag) {
        constexpr int HH = decltype(tag)::H;
        hipLaunchKernelGGL(permute_edges_kernel<HH>, dim3(grid_for(n, kBlock, 65536)), dim3(kBlock), 0, stream, perm,
                           src, n, scale, dst);
    });
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_edge_dot(int dtype, int H, int D, const int32_t* rows, const int32_t* col, int64_t n_edges,
                           const float* gf, const void* ff, float* out, hipStream_t stream) {
    if (n_edges == 0) return hipSuccess;
    const bool ok = dispatch_shape(dtype, H, D, [&](auto tag) {
        using Tag = decltype(tag);
        using T = typename Tag::type;
        using Gm = Geo<T, Tag::H, Tag::D>;
        constexpr int UMAX = (8 / Gm::NV) > 1 ? (8 / Gm::NV) : 1;
        constexpr int U = UMAX * Gm::P <= kWave ? UMAX : kWave / Gm::P;
        const int64_t waves = (n_edges + U * Gm::P - 1) / (U * Gm::P);
        hipLaunchKernelGGL((edge_dot_kernel<T, Tag::H, Tag::D>), dim3(grid_for(waves, kWavesPerBlock, edge_grid_cap())),
                           dim3(kBlock), 0, stream, rows, col, n_edges, gf, static_cast<const T*>(ff), out);
    });
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_softmax_backward(int H, const int32_t* row_ptr, int64_t n_rows, const float* alpha,
                                   const float* grad, float* out, float scale, const PlanView* plan,
                                   hipStream_t stream) {
    const bool ok = dispatch_heads(H, [&](auto tag) {
        constexpr int HH = decltype(tag)::H;
        if (plan)
            hipLaunchKernelGGL(softmax_bwd_segment_kernel<HH>,
                               dim3(grid_for(plan->seg_capacity, kWavesPerBlock, kSegmentGrid)), dim3(kBlock),
                               0, stream, alpha, grad, out, *plan, scale);
        // rows per wave: a multiple of the slots per wave, small enough to fill the device
        constexpr int slots = kWave / kSbG;
        int64_t rpw = (n_rows + kSbFillWaves - 1) / kSbFillWaves;
        rpw = (rpw + slots - 1) / slots * slots;
        rpw = rpw < slots ? slots : (rpw > kSbRowsPerWave ? kSbRowsPerWave : rpw);
        const int64_t waves = (n_rows + rpw - 1) / rpw;
        hipLaunchKernelGGL(softmax_bwd_short_kernel<HH>, dim3(grid_for(waves, kWavesPerBlock, INT32_MAX)),
                           dim3(kBlock), 0, stream, row_ptr, n_rows, alpha, grad, out,
                           plan ? plan->short_max : INT32_MAX, scale, (int)rpw);
        if (plan)
            hipLaunchKernelGGL(softmax_bwd_hub_kernel<HH>,
                               dim3(grid_for(plan->hubseg_capacity, 1, kSegmentGrid)), dim3(kBlock), 0, stream,
                               row_ptr, alpha, grad, out, *plan, scale);
    });
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gat
