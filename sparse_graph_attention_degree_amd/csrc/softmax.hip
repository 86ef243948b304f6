// Row-wise multi-head edge softmax (POPCORNBENCH l1_p6, the reference model: for
// every node and head, softmax over the node's edge slice of scores [E,H],
// computed as exp(x - max) / sum(exp(x - max))).
//
// The page's kernels map one thread to a (node, head) pair striding through the
// slice with stride H, or one block per node with shared-memory reductions.
// Here, by degree:
//  * short rows (the common case): a wave takes up to 64 consecutive rows; their scores
//    form one contiguous run, read in groups of whole rows (up to kBlkBudget floats,
//    16 consecutive per lane); per (row, head) maxima and sums combine through LDS
//    atomics that are exact in any order; one HBM round trip per group of rows.
//  * rows too long for the stage but not binned long (no plan, or a large
//    short_max): a 32-lane slot per row reads the row 32 values at a time (lane q:
//    edge q/H, head q%H), per-head max / sum are xor-shuffle trees over lanes q,
//    q^H, q^2H, ...; three passes: max, sum of exp, write.
//  * long rows and hub segments (the plan's segment table): a wave per segment,
//    streaming it in 1024-float chunks with a running (max, sum) per head; a row of
//    one chunk is written from registers.  Hub rows: a workgroup per hub segment
//    merges the row's segment (max, sum) states and writes alpha.
// A row's result does not depend on the rows around it (a batch of graphs gives
// every graph's rows the same bits as the graph alone): each (row, head) is
// reduced in an order fixed by the row, or with operations exact in any order.
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

// Rows per wave of the staged kernel (at most: fewer on graphs too small to fill the device).  64
// halves the waves where rows are short (c5's staged rows average 1.4 edges: 1198 against 1211 us
// for the call, c4 unchanged); at H = 16 the (row, head) tables would then take 32 KB of LDS per
// workgroup and cut the resident waves, so it stays at 32 there.
template <int H>
constexpr int blk_rows() { return H >= 16 ? 32 : 64; }
constexpr int64_t kSmFillWaves = 2048;
constexpr int kBlkBudget = 1024;   // floats per group (whole rows), 16 per lane

// Per-(row, head) maxima of a group combine with the LDS float max atomic (ds_max_f32: exact, so the
// same in any order).  Sums of exp(s - max) combine in fixed point: each term, in (0, 1], is
// truncated to a multiple of 1 / scale, so the sum is exact integer arithmetic, the same in any
// order.  A row of n edges sums to at least scale (its maximum contributes exactly 1), and the
// truncation moves the sum by less than n / scale relative to that.  Rows of up to kZ32Rows edges
// use 32-bit sums with scale 2^24 (n / scale <= 7.6e-6, 128 * 2^24 = 2^31 fits); longer ones (a
// group takes rows of up to 1024 / H edges) 64-bit sums with scale 2^31.
constexpr int kZ32Rows = 128;
template <bool Z32>
struct FixSum;
template <>
struct FixSum<true> {
    using type = unsigned;
    static constexpr float scale = 16777216.f;      // 2^24
    __device__ static type of(float p) { return (unsigned)(p * scale); }
};
template <>
struct FixSum<false> {
    using type = unsigned long long;
    static constexpr float scale = 2147483648.f;    // 2^31
    __device__ static type of(float p) { return (unsigned long long)(unsigned)(p * scale); }
};

// The H values of one (row, .) slot group from LDS, 16 or 8 bytes at a time (the slots of a row are
// consecutive and start at a multiple of H floats, so the vector reads are aligned).
template <int H>
__device__ __forceinline__ void read_heads(const float* p, float (&v)[H]) {
    if constexpr (H % 4 == 0) {
#pragma unroll
        for (int h = 0; h < H; h += 4) {
            const float4 q = *reinterpret_cast<const float4*>(p + h);
            v[h] = q.x;
            v[h + 1] = q.y;
            v[h + 2] = q.z;
            v[h + 3] = q.w;
        }
    } else if constexpr (H == 2) {
        const float2 q = *reinterpret_cast<const float2*>(p);
        v[0] = q.x;
        v[1] = q.y;
    } else {
#pragma unroll
        for (int h = 0; h < H; ++h) v[h] = p[h];
    }
}

// DPP move from the lane CTRL names; a lane whose source is outside its row, or whose row is not
// in ROWS, receives 0 (so the values must be >= 0 for the max below).
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_or0(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, true);
}

// Exclusive max-scan over the wave of non-negative values (lane 0 gets 0), in registers: shifts
// by 1, 2, 4 and 8 within each row of 16 lanes, then lane 15 of each row into the next row and
// lane 31 into the upper two rows, then a shift of the whole wave by one lane.
__device__ __forceinline__ int wave_max_scan_excl(int x) {
    x = max(x, dpp_or0<0x111, 0xF>(x));   // row_shr:1
    x = max(x, dpp_or0<0x112, 0xF>(x));   // row_shr:2
    x = max(x, dpp_or0<0x114, 0xF>(x));   // row_shr:4
    x = max(x, dpp_or0<0x118, 0xF>(x));   // row_shr:8
    x = max(x, dpp_or0<0x142, 0xA>(x));   // row_bcast:15, into rows 1 and 3
    x = max(x, dpp_or0<0x143, 0xC>(x));   // row_bcast:31, into rows 2 and 3
    return dpp_or0<0x138, 0xF>(x);        // wave_shr:1
}

// Rows with 0 < deg <= hi (hi * H <= kBlkBudget): a wave per rpw (<= blk_rows) consecutive rows, in
// groups of consecutive such rows (whole rows, at most kBlkBudget floats).  A row of another class
// (non-empty, deg > hi) ends a group, since its scores sit between the groups' runs.
//
// Lane l takes floats 16l .. 16l+15 of the group's run: 16 / H consecutive edges of all H heads,
// read with four 16-byte buffer loads straight into registers (a load past the run reads 0 and is
// masked).  The row of each edge comes from a table of the group's row starts in LDS (the row
// lanes mark their first edge; a max-scan over the lane's edges and over the lanes spreads the
// marks).  Then, per (row, head): the lane folds its own edges of one row (a running value that
// restarts where the row changes), and LDS atomics combine the lanes' parts -- a float max
// (exact), then the sum of exp(s - max) in fixed point (FixSum: exact integer adds) -- so a row's
// result is the same whatever rows share its group or lane.  alpha = exp(s - max) * (scale / sum)
// leaves through a per-wave LDS stage as 16-byte buffer stores of consecutive floats.
template <int H, bool Z32>
__global__ __launch_bounds__(kBlock) void softmax_block_kernel(const int32_t* __restrict__ row_ptr, int64_t n_rows,
                                                               const float* sc, float* out, int hi, int rpw) {
    using Fix = FixSum<Z32>;
    using ZT = typename Fix::type;
    constexpr int EPL = 16 / H;                // edges per lane
    constexpr int RIDB = kBlkBudget / H;       // edges per group, at most: bytes of the row table
    constexpr int NRH = blk_rows<H>() * H;     // (row, head) slots
    // Each wave's LDS area: the row table, the (row, head) maxima (then scale / sum) and the sums,
    // and, once a group's alpha is in registers, the same bytes as the 4 KB stage of its stores.
    constexpr int TAB = RIDB + NRH * 4 + NRH * (int)sizeof(ZT);
    constexpr int WB = TAB > kBlkBudget * 4 ? TAB : kBlkBudget * 4;
    __shared__ __align__(16) unsigned char wave_lds[kWavesPerBlock][WB];
    const int wv = threadIdx.x / kWave;
    unsigned char* rid_t = wave_lds[wv];
    float* mx = reinterpret_cast<float*>(wave_lds[wv] + RIDB);
    float* rzs = mx;
    ZT* zs = reinterpret_cast<ZT*>(wave_lds[wv] + RIDB + NRH * 4);
    float* stage = reinterpret_cast<float*>(wave_lds[wv]);
    const int lane = lane_id();
    const int64_t r0 = ((int64_t)blockIdx.x * kWavesPerBlock + wv) * rpw;
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
        // the group ends at the next breaker row or where the run would overflow kBlkBudget
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
        float x[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const gat_v4i a = __builtin_amdgcn_raw_buffer_load_b128(src, (lane * 16 + q * 4) * 4, 0, 0);
            x[4 * q] = __int_as_float(a.x);
            x[4 * q + 1] = __int_as_float(a.y);
            x[4 * q + 2] = __int_as_float(a.z);
            x[4 * q + 3] = __int_as_float(a.w);
        }
        const int nrows = j - i;
        wave_lds_handoff();   // the previous group's table reads come before these rewrites
        // clear the row table; reset the (row, head) slots
        if (lane * 16 < RIDB) *reinterpret_cast<uint4*>(rid_t + lane * 16) = make_uint4(0, 0, 0, 0);
        for (int t = lane; t < nrows * H; t += kWave) {
            mx[t] = -INFINITY;
            zs[t] = 0;
        }
        wave_lds_handoff();
        if (lane >= i && lane < j && deg > 0) rid_t[rb - base] = (unsigned char)(lane - i + 1);
        wave_lds_handoff();
        // rows of this lane's edges: marks max-scanned along the edges, then over the lanes (DPP)
        int rid[EPL];
        {
            unsigned char bt[EPL];
            if constexpr (EPL == 16) {
                const uint4 w = *reinterpret_cast<const uint4*>(rid_t + lane * 16);
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int k = 0; k < 16; ++k) bt[k] = (ww[k / 4] >> (8 * (k % 4))) & 0xff;
            } else if constexpr (EPL == 8) {
                const uint2 w = *reinterpret_cast<const uint2*>(rid_t + lane * 8);
#pragma unroll
                for (int k = 0; k < 8; ++k) bt[k] = ((k < 4 ? w.x : w.y) >> (8 * (k % 4))) & 0xff;
            } else if constexpr (EPL == 4) {
                const uint32_t w = *reinterpret_cast<const uint32_t*>(rid_t + lane * 4);
#pragma unroll
                for (int k = 0; k < 4; ++k) bt[k] = (w >> (8 * k)) & 0xff;
            } else if constexpr (EPL == 2) {
                const uint32_t w = *reinterpret_cast<const uint16_t*>(rid_t + lane * 2);
                bt[0] = w & 0xff;
                bt[1] = w >> 8;
            } else {
                bt[0] = rid_t[lane];
            }
            int run = 0;
#pragma unroll
            for (int k = 0; k < EPL; ++k) {
                run = bt[k] > run ? bt[k] : run;
                rid[k] = run;
            }
            const int excl = wave_max_scan_excl(run);
#pragma unroll
            for (int k = 0; k < EPL; ++k) rid[k] = (rid[k] > excl ? rid[k] : excl) - 1;
        }
        // per (row, head): the lane's own edges of one row folded (a running value that restarts
        // where the row changes), then an atomic max of the keys at the row's last edge in the lane
        {
            float run[H];
#pragma unroll
            for (int k = 0; k < EPL; ++k) {
                const bool valid = (lane * 16 + k * H) < len;
                const bool restart = k == 0 || rid[k] != rid[k - 1];
                const bool lastk = k == EPL - 1 || rid[k + 1] != rid[k] || (lane * 16 + (k + 1) * H) >= len;
#pragma unroll
                for (int h = 0; h < H; ++h) {
                    const float v = x[k * H + h];
                    run[h] = restart ? v : fmaxf(run[h], v);
                }
                // one branch for the H atomics of this edge (a branch per atomic costs more issue
                // slots than the atomics themselves)
                if (valid && lastk) {
                    float* mr = mx + rid[k] * H;
#pragma unroll
                    for (int h = 0; h < H; ++h) atomicMax(mr + h, run[h]);
                }
            }
        }
        wave_lds_handoff();
        // exp(s - max); its fixed-point sum per (row, head), folded the same way, then atomics
        {
            ZT run[H];
#pragma unroll
            for (int k = 0; k < EPL; ++k) {
                const bool valid = (lane * 16 + k * H) < len;
                const bool restart = k == 0 || rid[k] != rid[k - 1];
                const bool lastk = k == EPL - 1 || rid[k + 1] != rid[k] || (lane * 16 + (k + 1) * H) >= len;
                float m[H];
                read_heads<H>(mx + (valid ? rid[k] : 0) * H, m);
#pragma unroll
                for (int h = 0; h < H; ++h) {
                    const float p = valid ? exp_fast(x[k * H + h] - m[h]) : 0.f;
                    x[k * H + h] = p;
                    const ZT f = Fix::of(p);
                    run[h] = restart ? f : run[h] + f;
                }
                if (valid && lastk) {
                    ZT* zr = zs + rid[k] * H;
#pragma unroll
                    for (int h = 0; h < H; ++h) atomicAdd(zr + h, run[h]);
                }
            }
        }
        wave_lds_handoff();
        for (int t = lane; t < nrows * H; t += kWave) rzs[t] = Fix::scale / (float)zs[t];
        wave_lds_handoff();
#pragma unroll
        for (int k = 0; k < EPL; ++k) {
            const bool valid = (lane * 16 + k * H) < len;
            float r[H];
            read_heads<H>(rzs + (valid ? rid[k] : 0) * H, r);
#pragma unroll
            for (int h = 0; h < H; ++h) x[k * H + h] *= r[h];
        }
        // Stores through the stage: every lane puts its 16 consecutive floats into LDS, then stores
        // 16 bytes per instruction at consecutive positions, so one store instruction writes 1 KB
        // of consecutive floats.  Stored straight from registers, each instruction would write 64
        // pieces of 16 bytes 64 bytes apart (measured 20 % slower).  Piece t (16 bytes) of lane L
        // sits at slot 4 L + ((t + L / 4) & 3): every 16 lanes of a 16-byte LDS write, and of the
        // coalesced read, then touch 16 different bank groups.
        // A read-and-store past the group's run is skipped as a whole (a wave-uniform test).
        float4* st4 = reinterpret_cast<float4*>(stage);
        wave_lds_handoff();   // the tables' last reads come before the stage overwrites them
#pragma unroll
        for (int t = 0; t < 4; ++t)
            st4[4 * lane + ((t + (lane >> 2)) & 3)] = make_float4(x[4 * t], x[4 * t + 1], x[4 * t + 2], x[4 * t + 3]);
        wave_lds_handoff();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = q * kWave + lane;             // piece c of the group: lane c / 4, piece c % 4
            if (q * kWave * 4 < len) {
                const int L = c >> 2;
                const float4 v = st4[4 * L + (((c & 3) + (L >> 2)) & 3)];
                const gat_v4i a = {__float_as_int(v.x), __float_as_int(v.y), __float_as_int(v.z), __float_as_int(v.w)};
                __builtin_amdgcn_raw_buffer_store_b128(a, dst, c * 16, 0, 0);
            }
        }
        i = j;
    }
}

// Grid cap of the segment kernel (a wave per segment, striding past 2^16 waves).  The table's
// capacity counts every row that could be long (E / (short_max + 1) of them), several times the
// segments a power-law graph has, and the workgroups past the real count still cost dispatch time:
// at c4 (2^24 edges) 16384 workgroups took the kernel from 72 to 62 us; at c5 (2^26 edges, 74k
// segments) it made no difference, and smaller caps lost there (4096: +60 us).
constexpr int64_t kSoftmaxSegmentGrid = 16384;

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
    // The table is walked from its end: long rows first, then the hub segments from last to
    // first, so the hub scores read last (hub segment 0 onwards) are the first ones the alpha pass
    // reads again, while they may still be in the Infinity Cache.
    for (int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + wave; w < n_segs; w += n_waves) {
        const int4 sg = plan.segs[n_segs - 1 - w];
        const int64_t n = (int64_t)(sg.z - sg.y) * H;
        const float* seg = sc + (int64_t)sg.y * H;
        float m = -INFINITY, z = 0.f;
        // folds one chunk (cn floats in x, masked to -inf past the end) into (m, z)
        auto fold = [&](float(&x)[kSegRegs], int cn) {
            float cm = -INFINITY;
#pragma unroll
            for (int k = 0; k < kSegRegs; ++k) {
                if (lane >= cn - k * kWave) x[k] = -INFINITY;   // scalar bound: no per-k lane index kept
                cm = fmaxf(cm, x[k]);
            }
#pragma unroll
            for (int o = H; o < kWave; o <<= 1) cm = fmaxf(cm, shfl_xor(cm, o));
            const float mn = fmaxf(m, cm);   // finite: the chunk holds an element of this head
            float cz = 0.f;
#pragma unroll
            for (int k = 0; k < kSegRegs; ++k)
                if (k * kWave < cn) cz += exp_fast(x[k] - mn);   // exp(-inf) = 0 past the end
            z = z * exp_fast(m - mn) + cz;                         // m = -inf on the first chunk: z = cz
            m = mn;
        };
        // floats of the chunk at c0, 0 past the end (its loads then read 0 and move no data)
        auto chunk_len = [&](int64_t c0) {
            return opaque_uniform((int)(n - c0 <= 0 ? 0 : (n - c0 < kWaveChunk ? n - c0 : kWaveChunk)));
        };
        // A chunk's kSegRegs loads, all issued: those past the chunk's end read 0 and move no data.
        // No branch between them, so each lands in its own register of x and no copy has to wait.
        auto load_chunk = [&](float(&x)[kSegRegs], int64_t c0, int cn) {
            const __amdgpu_buffer_rsrc_t src = span(seg + c0, (int64_t)cn * 4);
            const int b = opaque(lane * 4);
#pragma unroll
            for (int k = 0; k < kSegRegs; ++k) x[k] = bload(src, b + k * kWave * 4);
        };
        float v[kSegRegs];
        int cv = chunk_len(0);
        load_chunk(v, 0, cv);
        if (n > kWaveChunk) {
            // Two chunk buffers: the next chunk's loads are in flight while the current one is
            // folded.  They are issued unconditionally (an empty chunk past the end at most), so
            // the compiler counts them exactly and waits only for the chunk it folds.  v holds the
            // chunk at c0 on entry to each pass.
            float u[kSegRegs];
            int64_t c0 = 0;
            do {
                const int cu = chunk_len(c0 + kWaveChunk);
                load_chunk(u, c0 + kWaveChunk, cu);
                __builtin_amdgcn_sched_barrier(0);   // the scheduler would sink the loads below the fold
                fold(v, cv);
                c0 += 2 * kWaveChunk;
                cv = chunk_len(c0);
                load_chunk(v, c0, cv);
                __builtin_amdgcn_sched_barrier(0);
                fold(u, cu);
            } while (c0 + kWaveChunk < n);
        }
        if (cv > 0) fold(v, cv);   // the last chunk (or the only one)
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
        // alpha of one chunk; the stores past the chunk's end are dropped
        auto store_chunk = [&](const float(&x)[kSegRegs], int64_t c0, int cn) {
            const __amdgpu_buffer_rsrc_t dst = span(dseg + c0, (int64_t)cn * 4);
            const int b = opaque(lane * 4);
#pragma unroll
            for (int k = 0; k < kSegRegs; ++k) bstore(dst, exp_fast(x[k] - m) * rz, b + k * kWave * 4);
        };
        if (n <= kWaveChunk) {
            // the segment is still in registers; only the stores that hold data are issued
            const __amdgpu_buffer_rsrc_t dst = span(dseg, (int64_t)cv * 4);
            const int b = opaque(lane * 4);
#pragma unroll
            for (int k = 0; k < kSegRegs; ++k)
                if (k * kWave < cv) bstore(dst, exp_fast(v[k] - m) * rz, b + k * kWave * 4);
            continue;
        }
        // A longer long row is read again, pipelined as above: the next chunk's loads are in
        // flight while the current one's alpha is computed and stored.
        {
            float u[kSegRegs];
            int64_t c0 = 0;
            cv = chunk_len(0);
            load_chunk(v, 0, cv);
            do {
                const int cu = chunk_len(c0 + kWaveChunk);
                load_chunk(u, c0 + kWaveChunk, cu);
                __builtin_amdgcn_sched_barrier(0);
                store_chunk(v, c0, cv);
                c0 += 2 * kWaveChunk;
                cv = chunk_len(c0);
                load_chunk(v, c0, cv);
                __builtin_amdgcn_sched_barrier(0);
                store_chunk(u, c0 - kWaveChunk, cu);
            } while (c0 < n);
        }
    }
}

constexpr int kHubBatch = 16;   // floats per thread per batch

// (m, z) states merge: m = max(m1, m2), z = z1 e^(m1 - m) + z2 e^(m2 - m); an empty state has
// m = -inf and contributes nothing.
__device__ __forceinline__ void merge_state(float& m, float& z, float m2, float z2) {
    const float mn = fmaxf(m, m2);
    z = (m == -INFINITY ? 0.f : z * exp_fast(m - mn)) + (m2 == -INFINITY ? 0.f : z2 * exp_fast(m2 - mn));
    m = mn;
}

// One workgroup per hub segment.  First the row's merged (max, sum) per head, from its segments'
// partial states: thread t takes head t % H and segments t / H, t / H + 256 / H, ..., merging them
// in that order, then block_head_reduce-style trees merge the threads' states (every workgroup
// of a row computes the same result in the same order).  Then alpha for this segment.  The
// scores of a segment are read in batches, all loads of a batch issued before the first store
// (out may alias sc, so the compiler would otherwise keep each load-exp-store in order).  With
// H >= 4 and 16-byte aligned arrays a segment's run starts on a 16-byte boundary, and threads move
// 4 consecutive floats at a time (heads (4t + j) % H, fixed per thread since 1024 is a multiple
// of H); otherwise one float at a time.
template <int H>
__global__ __launch_bounds__(kBlock) void softmax_hub_write_kernel(const int32_t* __restrict__ row_ptr,
                                                                   const float* sc, float* out, PlanView plan) {
    __shared__ float lm[kWavesPerBlock][H], lz[kWavesPerBlock][H];
    __shared__ float gM[H], gR[H];   // the row's max and 1 / sum per head
    const int t = threadIdx.x, lane = lane_id(), w = t / kWave;
    const int n_hub_segs = plan.counts[kNHubSegs];
    const bool wide = H >= 4 && ((reinterpret_cast<uintptr_t>(sc) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
    for (int s = blockIdx.x; s < n_hub_segs; s += gridDim.x) {
        const int4 sg = plan.segs[s];   // row, b, e, slot (= s)
        const int rb = row_ptr[sg.x], re = row_ptr[sg.x + 1];
        const int first = sg.w - (int)(((int64_t)sg.y - rb) / plan.seg_len);
        const int nseg = (int)(((int64_t)re - rb + plan.seg_len - 1) / plan.seg_len);
        // the row's state: per-thread merge over its segments, then the tree over the workgroup
        const int h = t % H;
        float m = -INFINITY, z = 0.f;
        for (int c = t / H; c < nseg; c += kBlock / H) {
            const float* pc = plan.partials + (int64_t)(first + c) * plan.state_floats;
            merge_state(m, z, pc[h], pc[H + h]);
        }
#pragma unroll
        for (int o = H; o < kWave; o <<= 1) {
            const float mo = shfl_xor(m, o), zo = shfl_xor(z, o);
            merge_state(m, z, mo, zo);
        }
        if (lane < H) {
            lm[w][lane] = m;
            lz[w][lane] = z;
        }
        __syncthreads();
        if (t < H) {
            float M = lm[0][t], Z = lz[0][t];
#pragma unroll
            for (int i = 1; i < kWavesPerBlock; ++i) merge_state(M, Z, lm[i][t], lz[i][t]);
            gM[t] = M;
            gR[t] = 1.f / Z;
        }
        __syncthreads();
        const int64_t beg = (int64_t)sg.y * H, end = (int64_t)sg.z * H;
        if (wide) {
            constexpr int NB = kHubBatch / 4;   // float4 per thread per batch
            const float4* s4 = reinterpret_cast<const float4*>(sc + beg);
            float4* o4 = reinterpret_cast<float4*>(out + beg);
            const int64_t n4 = (end - beg) / 4;   // H >= 4: whole float4s
            const int h0 = (4 * t) % H;
            float M[4], rz[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                M[j] = gM[(h0 + j) % H];
                rz[j] = gR[(h0 + j) % H];
            }
            for (int64_t f0 = t; f0 < n4; f0 += NB * kBlock) {
                float4 v[NB];
#pragma unroll
                for (int k = 0; k < NB; ++k) {
                    const int64_t f = f0 + (int64_t)k * kBlock;
                    v[k] = f < n4 ? s4[f] : make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
                for (int k = 0; k < NB; ++k) {
                    const int64_t f = f0 + (int64_t)k * kBlock;
                    if (f < n4)
                        o4[f] = make_float4(exp_fast(v[k].x - M[0]) * rz[0], exp_fast(v[k].y - M[1]) * rz[1],
                                            exp_fast(v[k].z - M[2]) * rz[2], exp_fast(v[k].w - M[3]) * rz[3]);
                }
            }
        } else {
            // kBlock is a multiple of H, so every element this thread touches has head t % H
            const float M = gM[h], rz = gR[h];
            for (int64_t i0 = beg + t; i0 < end; i0 += kHubBatch * kBlock) {
                float v[kHubBatch];
#pragma unroll
                for (int k = 0; k < kHubBatch; ++k) {
                    const int64_t i = i0 + (int64_t)k * kBlock;
                    v[k] = i < end ? sc[i] : 0.f;
                }
#pragma unroll
                for (int k = 0; k < kHubBatch; ++k) {
                    const int64_t i = i0 + (int64_t)k * kBlock;
                    if (i < end) out[i] = exp_fast(v[k] - M) * rz;
                }
            }
        }
        __syncthreads();   // gM / gR and lm / lz are rewritten for the next segment
    }
}

}  // namespace

hipError_t launch_softmax(int H, const int32_t* row_ptr, int64_t n_rows, const float* scores, float* out,
                          const PlanView* plan, hipStream_t stream) {
    const bool ok = dispatch_heads(H, [&](auto tag) {
        constexpr int HH = decltype(tag)::H;
        const int short_max = plan ? plan->short_max : INT32_MAX;
        const int staged = short_max < kBlkBudget / HH ? short_max : kBlkBudget / HH;   // rows the stage takes
        // Disjoint rows: the staged and slot kernels first, then the plan's segments (read from the
        // end of the table), then the hub alpha pass, which starts with the hub scores read last.
        int64_t rpw = (n_rows + kSmFillWaves - 1) / kSmFillWaves;   // enough waves to fill the device
        rpw = rpw < 1 ? 1 : (rpw > blk_rows<HH>() ? blk_rows<HH>() : rpw);
        const int64_t bwaves = (n_rows + rpw - 1) / rpw;
        if (staged <= kZ32Rows)
            hipLaunchKernelGGL((softmax_block_kernel<HH, true>), dim3(grid_for(bwaves, kWavesPerBlock, INT32_MAX)),
                               dim3(kBlock), 0, stream, row_ptr, n_rows, scores, out, staged, (int)rpw);
        else
            hipLaunchKernelGGL((softmax_block_kernel<HH, false>), dim3(grid_for(bwaves, kWavesPerBlock, INT32_MAX)),
                               dim3(kBlock), 0, stream, row_ptr, n_rows, scores, out, staged, (int)rpw);
        if (short_max > staged) {
            const int64_t waves = (n_rows + kSmRowsPerWave - 1) / kSmRowsPerWave;
            hipLaunchKernelGGL(softmax_short_kernel<HH>, dim3(grid_for(waves, kWavesPerBlock, INT32_MAX)),
                               dim3(kBlock), 0, stream, row_ptr, n_rows, scores, out, staged, short_max);
        }
        if (plan)
            hipLaunchKernelGGL(softmax_segment_kernel<HH>,
                               dim3(grid_for(plan->seg_capacity, kWavesPerBlock, kSoftmaxSegmentGrid)),
                               dim3(kBlock), 0, stream, scores, out, *plan);
        if (plan)
            hipLaunchKernelGGL(softmax_hub_write_kernel<HH>,
                               dim3(grid_for(plan->hubseg_capacity, 1, kSegmentGrid)), dim3(kBlock), 0, stream,
                               row_ptr, scores, out, *plan);
    });
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gat
