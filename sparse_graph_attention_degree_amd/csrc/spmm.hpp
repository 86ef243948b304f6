// Weighted neighbour aggregation in three flavours, one engine:
//   kAgg     out[i,h,:] = sum_e w[e,h] x[col[e],h,:]                  (POPCORNBENCH l1_p18)
//   kSoftAgg out[i,h,:] = sum_e softmax_row(s)[e,h] x[col[e],h,:]     (POPCORNBENCH l2_p37)
//   kLayer   as kSoftAgg with s[e,h] = scale <q[i,h,:], k[col[e],h,:]> computed on the fly
//
// A slot (G lanes, see common.hpp) walks a stream of chunks: SC consecutive edges of one
// row at a time.  A chunk's column ids (lanes q < SC) and scores (one dword per lane)
// arrive with two coalesced loads; the source rows are gathered U edges at a time, all U
// gathers issued before the first is used.  Right after a chunk's gathers are issued the
// slot issues the loads of its NEXT chunk (the next edges of the row, or the first edges
// of its next row), so the index/score round trip hides behind the gathers.
//
// Softmax is kept online per row and head: a chunk's maximum c (xor-shuffle tree over
// the lanes of one head) raises the running maximum m to m' = max(m, c); the running sum
// and the accumulators are rescaled by e^(m-m') (skipped when no lane's maximum moved),
// and each edge-head weight p = e^(s-m') is computed once, by the lane that loaded s,
// then moved to the lanes of its feature pieces with one ds_bpermute.  out = acc / z.
// In kLayer the score needs the gathered k row, so the maximum moves per group of U edges.
//
// A range result is the state (m[h], z[h], acc[h,:]); two states merge as
//   m = max(m1, m2), z = z1 e^(m1-m) + z2 e^(m2-m), acc = acc1 e^(m1-m) + acc2 e^(m2-m).
#pragma once

#include <math.h>

#include "kernels.hpp"

namespace gat {

template <typename T, int H, int D, int MODE>
struct Engine {
    using Gm = Geo<T, H, D>;
    static constexpr int G = Gm::G, P = Gm::P, NV = Gm::NV, EPP = Gm::EPP, LPH = Gm::LPH, SC = Gm::SC,
                         HD = Gm::HD;
    static constexpr int UMAX = (8 / NV) > 1 ? (8 / NV) : 1;
    static constexpr int U = SC < UMAX ? SC : UMAX;   // gathers in flight per lane per piece

    float acc[NV][EPP];
    float m_s, z_s;            // kSoftAgg: running max / partial sum, score layout (lane q: head q % H)
    float m_p[NV], z_p[NV];    // kLayer: piece layout (every lane of a head holds it)
    float qf[NV][EPP];         // kLayer: the row's query
    int hv[NV];                // head of piece v
    int off[NV];               // element offset of piece v inside a row
    int q, lane_base, es;

    __device__ __forceinline__ void init_lane(int lane) {
        q = lane % G;
        lane_base = lane - q;
        es = q / H;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int pv = v * G + q;
            hv[v] = pv / LPH;
            off[v] = pv * EPP;
        }
    }

    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
#pragma unroll
            for (int k = 0; k < EPP; ++k) acc[v][k] = 0.f;
            m_p[v] = -INFINITY;
            z_p[v] = 0.f;
        }
        m_s = -INFINITY;
        z_s = 0.f;
    }

    // Loads of one chunk [c, min(c+SC, e1)): scores (score layout) and column ids (lanes q < n).
    __device__ __forceinline__ void load_chunk(const int32_t* __restrict__ col, const float* __restrict__ sc, int c,
                                               int e1, float& s, int& cv) const {
        const int n = (e1 - c) < SC ? (e1 - c) : SC;
        s = 0.f;
        cv = 0;
        if (MODE != kLayer && es < n) s = sc[(int64_t)c * H + q];
        if (q < n) cv = col[c + q];
    }

    __device__ __forceinline__ void load_q(const T* __restrict__ qrow) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const uint4 t = ld16(qrow + off[v]);
            unpack<T>(t, qf[v]);
        }
    }

    __device__ __forceinline__ void fma_piece(int v, float w, const uint4& x) {
        float f[EPP];
        unpack<T>(x, f);
#pragma unroll
        for (int k = 0; k < EPP; ++k) acc[v][k] = fmaf(w, f[k], acc[v][k]);
    }

    __device__ __forceinline__ void scale_acc(int v, float c) {
#pragma unroll
        for (int k = 0; k < EPP; ++k) acc[v][k] *= c;
    }

    // ---- kAgg / kSoftAgg: consume chunk [c, min(c+SC, e1)) with its loaded (s, cv); after the
    // first gathers are issued, load the chunk at (nc, ne) into (s_n, cv_n) if nc < ne.
    __device__ __forceinline__ void consume_scores(const int32_t* __restrict__ col, const float* __restrict__ sc,
                                                   const T* __restrict__ feat, int c, int e1, float s, int cv,
                                                   int nc, int ne, float& s_n, int& cv_n) {
        const int n = (e1 - c) < SC ? (e1 - c) : SC;
        float p;
        if constexpr (MODE == kSoftAgg) {
            const float sv = es < n ? s : -INFINITY;
            float cm = sv;
#pragma unroll
            for (int k = H; k < G; k <<= 1) cm = fmaxf(cm, shfl_xor(cm, k));
            const float mo = m_s;
            const float mn = fmaxf(mo, cm);
            const float corr = exp_fast(mo - mn);   // 0 on the row's first chunk
            m_s = mn;
            p = es < n ? exp_fast(sv - mn) : 0.f;
            z_s = fmaf(z_s, corr, p);
            if (__any(mo != -INFINITY && corr != 1.f)) {
#pragma unroll
                for (int v = 0; v < NV; ++v) scale_acc(v, shfl(corr, lane_base + hv[v]));
            }
        } else {
            p = es < n ? s : 0.f;
        }
#pragma unroll
        for (int jb = 0; jb < SC; jb += U) {
            if (jb >= n) break;
            uint4 x[U][NV];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = jb + u;
                const int cj = shfl(cv, lane_base + j);
                const T* src = feat + (int64_t)cj * HD;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    if (j < n) x[u][v] = ld16(src + off[v]);
                    else x[u][v] = make_uint4(0u, 0u, 0u, 0u);
                }
            }
            if (jb == 0 && nc < ne) load_chunk(col, sc, nc, ne, s_n, cv_n);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = jb + u;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const float w = shfl(p, lane_base + j * H + hv[v]);
                    if (j < n) fma_piece(v, w, x[u][v]);
                }
            }
        }
    }

    // ---- kLayer: consume chunk [c, min(c+SC, e1)) with its column ids cv (query in qf); after the
    // first gathers are issued, load the column ids of the chunk at (nc, ne) into cv_n.
    __device__ __forceinline__ void consume_layer(const int32_t* __restrict__ col, const T* __restrict__ kf,
                                                  const T* __restrict__ vf, float scale, int c, int e1, int cv,
                                                  int nc, int ne, int& cv_n) {
        const int n = (e1 - c) < SC ? (e1 - c) : SC;
#pragma unroll
        for (int jb = 0; jb < SC; jb += U) {
            if (jb >= n) break;
            uint4 kx[U][NV], vx[U][NV];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = jb + u;
                const int cj = shfl(cv, lane_base + j);
                const int64_t base = (int64_t)cj * HD;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    if (j < n) {
                        kx[u][v] = ld16(kf + base + off[v]);
                        vx[u][v] = ld16(vf + base + off[v]);
                    } else {
                        kx[u][v] = make_uint4(0u, 0u, 0u, 0u);
                        vx[u][v] = make_uint4(0u, 0u, 0u, 0u);
                    }
                }
            }
            if (jb == 0 && nc < ne) {
                float unused;
                load_chunk(col, nullptr, nc, ne, unused, cv_n);
            }
            float s[U][NV];
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    float f[EPP];
                    unpack<T>(kx[u][v], f);
                    float d = 0.f;
#pragma unroll
                    for (int k = 0; k < EPP; ++k) d = fmaf(qf[v][k], f[k], d);
#pragma unroll
                    for (int o = 1; o < LPH; o <<= 1) d += shfl_xor(d, o);
                    s[u][v] = (jb + u < n) ? d * scale : -INFINITY;
                }
            }
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                float mx = s[0][v];
#pragma unroll
                for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u][v]);
                const float mn = fmaxf(m_p[v], mx);
                const float corr = exp_fast(m_p[v] - mn);
                m_p[v] = mn;
                z_p[v] *= corr;
                scale_acc(v, corr);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float pw = exp_fast(s[u][v] - mn);
                    z_p[v] += pw;
                    fma_piece(v, pw, vx[u][v]);
                }
            }
        }
    }

    // Sum the per-lane partial sums of each head (kSoftAgg; all slot lanes must call).
    __device__ __forceinline__ void finish() {
        if constexpr (MODE == kSoftAgg) {
#pragma unroll
            for (int k = H; k < G; k <<= 1) z_s += shfl_xor(z_s, k);
        }
    }

    // max / sum of piece v's head (kSoftAgg converts from score layout; all slot lanes must call)
    __device__ __forceinline__ float m_piece(int v) const {
        if constexpr (MODE == kSoftAgg) return shfl(m_s, lane_base + hv[v]);
        else return m_p[v];
    }
    __device__ __forceinline__ float z_piece(int v) const {
        if constexpr (MODE == kSoftAgg) return shfl(z_s, lane_base + hv[v]);
        else return z_p[v];
    }

    // Final output of a whole row: acc / z (acc for kAgg); +0.0 for a row without edges.
    __device__ __forceinline__ void store_row(float* __restrict__ out_row, bool nonempty) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float inv = 1.f;
            if constexpr (MODE != kAgg) {
                const float z = z_piece(v);
                inv = nonempty ? 1.f / z : 0.f;
            }
#pragma unroll
            for (int k = 0; k < EPP; k += 4)
                st16(out_row + off[v] + k, acc[v][k] * inv, acc[v][k + 1] * inv, acc[v][k + 2] * inv,
                     acc[v][k + 3] * inv);
        }
    }

    __device__ __forceinline__ void store_zero_row(float* __restrict__ out_row) {
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int k = 0; k < EPP; k += 4) st16(out_row + off[v] + k, 0.f, 0.f, 0.f, 0.f);
    }

    // Range state into LDS: m[H], z[H], acc[HD] (all slot lanes must call).
    __device__ __forceinline__ void store_state(float* lds) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            if constexpr (MODE != kAgg) {
                const float m = m_piece(v), z = z_piece(v);
                if ((v * G + q) % LPH == 0) {
                    lds[hv[v]] = m;
                    lds[H + hv[v]] = z;
                }
            }
#pragma unroll
            for (int k = 0; k < EPP; k += 4)
                *reinterpret_cast<float4*>(lds + 2 * H + off[v] + k) =
                    make_float4(acc[v][k], acc[v][k + 1], acc[v][k + 2], acc[v][k + 3]);
        }
    }

    // Whole range [b, e) of one row as one chunk stream (segment kernels).
    __device__ __forceinline__ void run_range(const int32_t* __restrict__ col, const float* __restrict__ sc,
                                              const T* __restrict__ qrow, const T* __restrict__ kf,
                                              const T* __restrict__ vf, float scale, int b, int e) {
        reset();
        if (b >= e) return;
        float s = 0.f;
        int cv = 0;
        load_chunk(col, sc, b, e, s, cv);
        if constexpr (MODE == kLayer) load_q(qrow);
        for (int c = b; c < e; c += SC) {
            float s_n = 0.f;
            int cv_n = 0;
            if constexpr (MODE == kLayer) consume_layer(col, kf, vf, scale, c, e, cv, c + SC, e, cv_n);
            else consume_scores(col, sc, vf, c, e, s, cv, c + SC, e, s_n, cv_n);
            s = s_n;
            cv = cv_n;
        }
        finish();
    }
};

// ---------------------------------------------------------------------------------------------
// Short rows: a wave takes kRowsPerWave consecutive rows and each slot a contiguous block of
// RS = kRowsPerWave / P of them, so a slot's edges form one contiguous run that it walks as a
// single chunk stream (prefetching across row boundaries).  Rows with deg > short_max belong
// to the segment kernel and are skipped; short_max = INT_MAX without a plan.
constexpr int kRowsPerWave = 32;

template <typename T, int H, int D, int MODE>
__global__ __launch_bounds__(kBlock) void spmm_short_kernel(const int32_t* __restrict__ row_ptr,
                                                            const int32_t* __restrict__ col, int64_t n_rows,
                                                            const float* __restrict__ sc, const T* __restrict__ qf,
                                                            const T* __restrict__ kf, const T* __restrict__ vf,
                                                            float scale, float* __restrict__ out, int short_max) {
    using E = Engine<T, H, D, MODE>;
    constexpr int P = E::P, G = E::G, HD = E::HD, SC = E::SC;
    constexpr int RS = kRowsPerWave / P;   // rows per slot (<= G/2)
    static_assert(RS + 1 <= G, "a slot holds its rows' row_ptr entries");
    const int lane = lane_id();
    const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    const int64_t wb = wave * kRowsPerWave;
    if (wb >= n_rows) return;
    E eng;
    eng.init_lane(lane);
    const int q = eng.q, lb = eng.lane_base;
    const int64_t row0 = wb + (int64_t)(lane / G) * RS;
    int rpv = 0;
    if (q <= RS && row0 + q <= n_rows) rpv = row_ptr[row0 + q];

    // Row it of this slot: [e0, e1), or empty when it is not ours (past the end, or binned long).
    auto bounds = [&](int it, int& e0, int& e1) {
        e0 = shfl(rpv, lb + it);
        e1 = shfl(rpv, lb + it + 1);
        if (!(row0 + it < n_rows && e1 - e0 <= short_max)) e1 = e0;
    };
    // Rows of ours with no edges get +0.0 now; the stream below visits only non-empty rows.
    for (int it = 0; it < RS; ++it) {
        const int a = shfl(rpv, lb + it), b = shfl(rpv, lb + it + 1);
        if (row0 + it < n_rows && a == b) eng.store_zero_row(out + (row0 + it) * HD);
    }
    // First non-empty row at or after `it` (RS when none).
    auto next_row = [&](int it, int& e0, int& e1) {
        for (; it < RS; ++it) {
            bounds(it, e0, e1);
            if (e1 > e0) break;
        }
        return it;
    };

    int e0 = 0, e1 = 0;
    int it = next_row(0, e0, e1);
    if (it >= RS) return;
    float s = 0.f;
    int cv = 0;
    eng.reset();
    eng.load_chunk(col, sc, e0, e1, s, cv);
    if constexpr (MODE == kLayer) eng.load_q(qf + (row0 + it) * HD);
    int c = e0;
    while (true) {
        // successor chunk: the rest of this row, or the first chunk of the next non-empty row
        int nit = it, nc = c + SC, ne = e1;
        if (nc >= e1) {
            int f0 = 0, f1 = 0;
            nit = next_row(it + 1, f0, f1);
            nc = f0;
            ne = nit < RS ? f1 : f0;
        }
        float s_n = 0.f;
        int cv_n = 0;
        if constexpr (MODE == kLayer) eng.consume_layer(col, kf, vf, scale, c, e1, cv, nc, ne, cv_n);
        else eng.consume_scores(col, sc, vf, c, e1, s, cv, nc, ne, s_n, cv_n);
        if (nit != it) {
            eng.finish();
            eng.store_row(out + (row0 + it) * HD, true);
            if (nit >= RS) break;
            eng.reset();
            if constexpr (MODE == kLayer) eng.load_q(qf + (row0 + nit) * HD);
            e1 = ne;
        }
        it = nit;
        c = nc;
        s = s_n;
        cv = cv_n;
    }
}

// ---------------------------------------------------------------------------------------------
// Long rows and hub segments: one 256-thread workgroup per segment of the plan's segment table
// (persistent grid, counts read on the device).  The 4*P slots split the segment's edges into
// contiguous sub-ranges, leave their states in LDS, and the workgroup merges them.  A long row
// (slot < 0) is written out; a hub segment's state goes to the plan's partial buffer.
template <typename T, int H, int D, int MODE>
__global__ __launch_bounds__(kBlock) void spmm_segment_kernel(const int32_t* __restrict__ col,
                                                              const float* __restrict__ sc,
                                                              const T* __restrict__ qf, const T* __restrict__ kf,
                                                              const T* __restrict__ vf, float scale,
                                                              float* __restrict__ out, PlanView plan) {
    using E = Engine<T, H, D, MODE>;
    constexpr int NS = kWavesPerBlock * E::P;   // slots per workgroup
    constexpr int HD = E::HD;
    constexpr int SS = HD + 2 * H;              // floats per state
    __shared__ __align__(16) float lds[NS * SS];
    const int lane = lane_id();
    const int gs = (threadIdx.x / kWave) * E::P + lane / E::G;
    const int n_segs = plan.counts[kNSegs];
    E eng;
    eng.init_lane(lane);
    for (int s = blockIdx.x; s < n_segs; s += gridDim.x) {
        const int4 sg = plan.segs[s];   // row, e_begin, e_end, slot
        const int64_t len = (int64_t)sg.z - sg.y;
        const int b = sg.y + (int)(len * gs / NS);
        const int e = sg.y + (int)(len * (gs + 1) / NS);
        eng.run_range(col, sc, qf + (int64_t)sg.x * HD, kf, vf, scale, b, e);
        eng.store_state(lds + gs * SS);
        __syncthreads();
        float* prt = sg.w >= 0 ? plan.partials + (int64_t)sg.w * plan.state_floats : nullptr;
        for (int el = threadIdx.x; el < HD; el += kBlock) {
            const int h = el / D;
            float M = -INFINITY, Z = 0.f, A = 0.f;
            if constexpr (MODE != kAgg) {
#pragma unroll
                for (int i = 0; i < NS; ++i) M = fmaxf(M, lds[i * SS + h]);
            }
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                float w = 1.f;
                if constexpr (MODE != kAgg) {
                    const float mi = lds[i * SS + h];
                    w = (mi == -INFINITY) ? 0.f : exp_fast(mi - M);
                    Z = fmaf(lds[i * SS + H + h], w, Z);
                }
                A = fmaf(lds[i * SS + 2 * H + el], w, A);
            }
            if (prt == nullptr) {
                out[(int64_t)sg.x * HD + el] = (MODE == kAgg) ? A : A / Z;
            } else {
                prt[2 * H + el] = A;
                if (el % D == 0) {
                    prt[h] = M;
                    prt[H + h] = Z;
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------------------------
// Hub rows: merge the states of a row's segments and write the row.
template <int MODE>
__global__ __launch_bounds__(kBlock) void spmm_hub_merge_kernel(float* __restrict__ out, int H, int D,
                                                                PlanView plan) {
    const int HD = H * D;
    const int n_hubs = plan.counts[kNHubs];
    for (int hb = blockIdx.x; hb < n_hubs; hb += gridDim.x) {
        const int4 hr = plan.hubs[hb];   // row, first segment, n segments
        for (int el = threadIdx.x; el < HD; el += kBlock) {
            const int h = el / D;
            const float* p0 = plan.partials + (int64_t)hr.y * plan.state_floats;
            float M = -INFINITY, Z = 0.f, A = 0.f;
            if (MODE != kAgg)
                for (int c = 0; c < hr.z; ++c) M = fmaxf(M, p0[(int64_t)c * plan.state_floats + h]);
            for (int c = 0; c < hr.z; ++c) {
                const float* pc = p0 + (int64_t)c * plan.state_floats;
                float w = 1.f;
                if (MODE != kAgg) {
                    w = (pc[h] == -INFINITY) ? 0.f : exp_fast(pc[h] - M);
                    Z = fmaf(pc[H + h], w, Z);
                }
                A = fmaf(pc[2 * H + el], w, A);
            }
            out[(int64_t)hr.x * HD + el] = (MODE == kAgg) ? A : A / Z;
        }
    }
}

template <int MODE>
hipError_t launch_spmm_mode(int dtype, int H, int D, const int32_t* row_ptr, const int32_t* col, int64_t n_rows,
                            const float* sc, const void* q, const void* k, const void* v, float scale,
                            float* out, const PlanView* plan, hipStream_t stream) {
    const bool ok = dispatch_shape(dtype, H, D, [&](auto tag) {
        using Tag = decltype(tag);
        using T = typename Tag::type;
        constexpr int HH = Tag::H, DD = Tag::D;
        const T* qt = static_cast<const T*>(q);
        const T* kt = static_cast<const T*>(k);
        const T* vt = static_cast<const T*>(v);
        if (plan)
            hipLaunchKernelGGL((spmm_segment_kernel<T, HH, DD, MODE>),
                               dim3(grid_for(plan->seg_capacity, 1, kPersistentBlocks)), dim3(kBlock), 0, stream,
                               col, sc, qt, kt, vt, scale, out, *plan);
        const int64_t waves = (n_rows + kRowsPerWave - 1) / kRowsPerWave;
        const unsigned blocks = grid_for(waves, kWavesPerBlock, INT32_MAX);
        hipLaunchKernelGGL((spmm_short_kernel<T, HH, DD, MODE>), dim3(blocks), dim3(kBlock), 0, stream, row_ptr,
                           col, n_rows, sc, qt, kt, vt, scale, out, plan ? plan->short_max : INT32_MAX);
    });
    if (!ok) return hipErrorInvalidValue;
    if (plan)
        hipLaunchKernelGGL(spmm_hub_merge_kernel<MODE>, dim3(grid_for(plan->hub_capacity, 1, kPersistentBlocks)),
                           dim3(kBlock), 0, stream, out, H, D, *plan);
    return hipGetLastError();
}

}  // namespace gat
