// Weighted neighbour aggregation in three flavours, one engine:
//   kAgg     out[i,h,:] = sum_e w[e,h] x[col[e],h,:]                  (POPCORNBENCH l1_p18)
//   kSoftAgg out[i,h,:] = sum_e softmax_row(s)[e,h] x[col[e],h,:]     (POPCORNBENCH l2_p37)
//   kLayer   as kSoftAgg with s[e,h] = scale <q[i,h,:], k[col[e],h,:]> computed on the fly
//
// A slot (G lanes, see common.hpp) walks a stream of chunks: SC consecutive edges of one
// row at a time.  A chunk's column ids and scores (one dword per lane) arrive with two
// coalesced loads; the source rows are gathered U edges at a time, all U gathers issued
// before the first is used.  Before a chunk's gathers are issued the slot issues the loads
// of its NEXT chunk (the next edges of the row, or the first edges of its next row; in
// kLayer also that row's query), so their round trip hides behind the gathers and the
// wait for the gathers never waits on a load issued after them.
//
// Softmax is kept online per row and head: a chunk's maximum c (xor-shuffle tree over
// the lanes of one head) raises the running maximum m to m' = max(m, c); the running sum
// and the accumulators are rescaled by e^(m-m') (skipped when no lane's maximum moved),
// and each edge-head weight p = e^(s-m') is computed once, by the lane that loaded s.
// The chunk's weights (transposed to [head][edge]) and column ids are staged in a small
// per-slot LDS area; each lane then reads its head's SC weights and the SC column ids with
// vector LDS reads at immediate offsets.  out = acc / z.
// In kLayer the score needs the gathered k row, so the maximum moves per group of U edges.
//
// Steps past a chunk's end use a column of the chunk (lanes past the end hold a clamped
// column id) with weight 0, and each step's guard is a wave-uniform branch.
//
// A range result is the state (m[h], z[h], acc[h,:]); two states merge as
//   m = max(m1, m2), z = z1 e^(m1-m) + z2 e^(m2-m), acc = acc1 e^(m1-m) + acc2 e^(m2-m).
#pragma once

#include <math.h>

#include <type_traits>

#include "kernels.hpp"

namespace gat {

// Score dwords each lane loads per chunk: a chunk is kChunkLoads * G/H edges.
constexpr int kChunkLoads = 1;

template <typename T, int H, int D, int MODE, class TAB, int GMAX = kWave>
struct Engine {
    using Gm = Geo<T, H, D, GMAX>;
    static constexpr int G = Gm::G, P = Gm::P, NV = Gm::NV, EPP = Gm::EPP, LPH = Gm::LPH, HD = Gm::HD,
                         RB = Gm::RB;
    static constexpr int SM = kChunkLoads;          // score loads per lane per chunk
    static constexpr int SC1 = Gm::SC;              // edges per score load (G/H)
    static constexpr int SC = SM * SC1;             // edges per chunk
    static constexpr int CM = (SC + G - 1) / G;     // column-id loads per lane per chunk
    static constexpr int UMAX = (8 * SM / NV) > 1 ? (8 * SM / NV) : 1;
    static constexpr int U = SC < UMAX ? SC : UMAX;   // gathers in flight per lane per piece
    static constexpr int UL = U;                       // kLayer: edges per group (a k and a v row each)

    float acc[NV][EPP];
    float m_s, z_s;            // kSoftAgg: running max / partial sum, score layout (lane q: head q % H)
    float m_p[NV], z_p[NV];    // kLayer: piece layout (every lane of a head holds it)
    float qf[NV][EPP];         // kLayer: the row's query
    int hv[NV];                // head of piece v
    int off[NV];               // element offset of piece v inside a row
    int q, lane_base, es;
    float* stage;              // this slot's LDS staging area: weights [H][SC], then column ids [SC]

    static constexpr int kStage = H * SC + SC;   // floats of staging per slot

    __device__ __forceinline__ void init_lane(int lane, float* slot_stage) {
        stage = slot_stage;
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

    __device__ __forceinline__ uint4 gather(const TAB& tab, int r, int v) const {
        return tab.row16(r, (uint32_t)off[v] * (uint32_t)sizeof(T));
    }

    // Loads of one chunk [c, min(c+SC, e1)): scores (score layout, load k covers edges
    // k*SC1 + q/H) and column ids (load k: edge k*G + q, clamped to the chunk's last edge, so
    // steps past the chunk's end gather a row of the chunk).
    __device__ __forceinline__ void load_chunk(const int32_t* __restrict__ col, const float* __restrict__ sc, int c,
                                               int e1, float (&s)[SM], int (&cv)[CM]) const {
        const int n = (e1 - c) < SC ? (e1 - c) : SC;
#pragma unroll
        for (int k = 0; k < SM; ++k) {
            s[k] = 0.f;
            if (MODE != kLayer && k * SC1 + es < n) s[k] = sc[(int64_t)(c + k * SC1) * H + q];
        }
#pragma unroll
        for (int k = 0; k < CM; ++k) {
            const int i = k * G + q;
            cv[k] = col[c + (i < n ? i : n - 1)];
        }
    }

    __device__ __forceinline__ void load_q_raw(const T* __restrict__ qrow, uint4 (&raw)[NV]) const {
#pragma unroll
        for (int v = 0; v < NV; ++v) raw[v] = ld16(qrow + off[v]);
    }

    __device__ __forceinline__ void set_q(const uint4 (&raw)[NV]) {
#pragma unroll
        for (int v = 0; v < NV; ++v) unpack<T>(raw[v], qf[v]);
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

    // ---- kAgg / kSoftAgg: consume chunk [c, min(c+SC, e1)) with its loaded (s, cv); first issue
    // the loads of the chunk at (nc, ne) into (s_n, cv_n) when nc < ne.
    __device__ __forceinline__ void consume_scores(const int32_t* __restrict__ col, const float* __restrict__ sc,
                                                   const TAB& vt, int c, int e1, const float (&s)[SM],
                                                   const int (&cv)[CM], int nc, int ne, float (&s_n)[SM],
                                                   int (&cv_n)[CM]) {
        const int n = (e1 - c) < SC ? (e1 - c) : SC;
        float p[SM];
        if constexpr (MODE == kSoftAgg) {
            float sv[SM];
            float cm = -INFINITY;
#pragma unroll
            for (int k = 0; k < SM; ++k) {
                sv[k] = k * SC1 + es < n ? s[k] : -INFINITY;
                cm = fmaxf(cm, sv[k]);
            }
#pragma unroll
            for (int k = H; k < G; k <<= 1) cm = fmaxf(cm, shfl_xor(cm, k));
            const float mo = m_s;
            const float mn = fmaxf(mo, cm);
            const float corr = exp_fast(mo - mn);   // 0 on the row's first chunk
            m_s = mn;
            float ps = 0.f;
#pragma unroll
            for (int k = 0; k < SM; ++k) {
                p[k] = k * SC1 + es < n ? exp_fast(sv[k] - mn) : 0.f;
                ps += p[k];
            }
            z_s = fmaf(z_s, corr, ps);
            if (__any(mo != -INFINITY && corr != 1.f)) {
#pragma unroll
                for (int v = 0; v < NV; ++v) scale_acc(v, shfl(corr, lane_base + hv[v]));
            }
        } else {
#pragma unroll
            for (int k = 0; k < SM; ++k) p[k] = k * SC1 + es < n ? s[k] : 0.f;
        }
        // weights transposed to [head][edge] and column ids into the slot's LDS area, which the
        // slot's lanes read back below (and read for the previous chunk before this rewrite).
        // Staged before the next chunk's loads are issued, so waiting for (s, cv) never waits
        // on them.
        wave_lds_handoff();
#pragma unroll
        for (int k = 0; k < SM; ++k) stage[(q % H) * SC + k * SC1 + es] = p[k];
#pragma unroll
        for (int k = 0; k < CM; ++k)
            if (k * G + q < SC) reinterpret_cast<int*>(stage)[H * SC + k * G + q] = cv[k];
        wave_lds_handoff();
        if (nc < ne) load_chunk(col, sc, nc, ne, s_n, cv_n);
#pragma unroll
        for (int jb = 0; jb < SC; jb += U) {
            if (!__any(jb < n)) break;
            int cj[U];
#pragma unroll
            for (int u = 0; u < U; ++u) cj[u] = reinterpret_cast<const int*>(stage)[H * SC + jb + u];
            uint4 x[U][NV];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (u == 0 || __any(jb + u < n)) {
#pragma unroll
                    for (int v = 0; v < NV; ++v) x[u][v] = gather(vt, cj[u], v);
                }
            }
            float w[U][NV];
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int u = 0; u < U; ++u) w[u][v] = stage[hv[v] * SC + jb + u];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (u == 0 || __any(jb + u < n)) {
#pragma unroll
                    for (int v = 0; v < NV; ++v) fma_piece(v, w[u][v], x[u][v]);
                }
            }
        }
    }

    // ---- kLayer: consume chunk [c, min(c+SC, e1)) with its column ids cv (query in qf); first
    // issue the column ids of the chunk at (nc, ne) into cv_n when nc < ne, and the query row
    // qn into qraw_n when qn is not null.
    __device__ __forceinline__ void consume_layer(const int32_t* __restrict__ col, const TAB& kt, const TAB& vt,
                                                  float scale, int c, int e1, const int (&cv)[CM], int nc, int ne,
                                                  int (&cv_n)[CM], const T* __restrict__ qn, uint4 (&qraw_n)[NV]) {
        const int n = (e1 - c) < SC ? (e1 - c) : SC;
        // column ids into the slot's LDS area for every lane of the slot (see consume_scores)
        wave_lds_handoff();
#pragma unroll
        for (int k = 0; k < CM; ++k)
            if (k * G + q < SC) reinterpret_cast<int*>(stage)[H * SC + k * G + q] = cv[k];
        wave_lds_handoff();
        if (nc < ne) {
            float unused[SM];
            load_chunk(col, nullptr, nc, ne, unused, cv_n);
        }
        if (qn != nullptr) load_q_raw(qn, qraw_n);
#pragma unroll
        for (int jb = 0; jb < SC; jb += UL) {
            if (!__any(jb < n)) break;
            int cj[UL];
#pragma unroll
            for (int u = 0; u < UL; ++u) cj[u] = reinterpret_cast<const int*>(stage)[H * SC + jb + u];
            uint4 kx[UL][NV], vx[UL][NV];
#pragma unroll
            for (int u = 0; u < UL; ++u) {
                if (u == 0 || __any(jb + u < n)) {
#pragma unroll
                    for (int v = 0; v < NV; ++v) {
                        kx[u][v] = gather(kt, cj[u], v);
                        vx[u][v] = gather(vt, cj[u], v);
                    }
                }
            }
            float s[UL][NV];
#pragma unroll
            for (int u = 0; u < UL; ++u) {
                const bool live = u == 0 || __any(jb + u < n);
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    s[u][v] = -INFINITY;
                    if (live) {
                        float f[EPP];
                        unpack<T>(kx[u][v], f);
                        float d = 0.f;
#pragma unroll
                        for (int k = 0; k < EPP; ++k) d = fmaf(qf[v][k], f[k], d);
                        d = group_sum<LPH>(d);
                        if (jb + u < n) s[u][v] = d * scale;
                    }
                }
            }
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                float mx = s[0][v];
#pragma unroll
                for (int u = 1; u < UL; ++u) mx = fmaxf(mx, s[u][v]);
                const float mn = fmaxf(m_p[v], mx);
                const float corr = exp_fast(m_p[v] - mn);
                m_p[v] = mn;
                z_p[v] *= corr;
                scale_acc(v, corr);
#pragma unroll
                for (int u = 0; u < UL; ++u) {
                    if (u == 0 || __any(jb + u < n)) {
                        const float pw = exp_fast(s[u][v] - mn);
                        z_p[v] += pw;
                        fma_piece(v, pw, vx[u][v]);
                    }
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

    // store_row for 16-bit features, through the slot's LDS row (HD floats): a lane's EPP = 8
    // floats of a piece are 32 bytes, so stored straight from registers every instruction would
    // write 16-byte pieces 32 bytes apart.  Each lane writes its pieces into LDS, then every
    // instruction stores 16 bytes per lane at consecutive positions.
    __device__ __forceinline__ void store_row_lds(float* __restrict__ out_row, float* row_lds, bool nonempty) {
        static_assert(EPP == 8, "16-bit features");
        wave_lds_handoff();   // the slot's reads of its previous row come before these writes
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float inv = 1.f;
            if constexpr (MODE != kAgg) {
                const float z = z_piece(v);
                inv = nonempty ? 1.f / z : 0.f;
            }
            float4* w = reinterpret_cast<float4*>(row_lds + off[v]);
            w[0] = make_float4(acc[v][0] * inv, acc[v][1] * inv, acc[v][2] * inv, acc[v][3] * inv);
            w[1] = make_float4(acc[v][4] * inv, acc[v][5] * inv, acc[v][6] * inv, acc[v][7] * inv);
        }
        wave_lds_handoff();
#pragma unroll
        for (int j = 0; j < 2 * NV; ++j) {
            const int e = (j * G + q) * 4;
            const float4 x = *reinterpret_cast<const float4*>(row_lds + e);
            st16(out_row + e, x.x, x.y, x.z, x.w);
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
                                              const T* __restrict__ qrow, const TAB& kt, const TAB& vt, float scale,
                                              int b, int e) {
        reset();
        if (b >= e) return;
        float s[SM];
        int cv[CM];
        load_chunk(col, sc, b, e, s, cv);
        if constexpr (MODE == kLayer) {
            uint4 raw[NV];
            load_q_raw(qrow, raw);
            set_q(raw);
        }
        for (int c = b; c < e; c += SC) {
            float s_n[SM] = {};
            int cv_n[CM] = {};
            if constexpr (MODE == kLayer) {
                uint4 unused[NV] = {};
                consume_layer(col, kt, vt, scale, c, e, cv, c + SC, e, cv_n, nullptr, unused);
            } else {
                consume_scores(col, sc, vt, c, e, s, cv, c + SC, e, s_n, cv_n);
            }
#pragma unroll
            for (int k = 0; k < SM; ++k) s[k] = s_n[k];
#pragma unroll
            for (int k = 0; k < CM; ++k) cv[k] = cv_n[k];
        }
        finish();
    }
};

// ---------------------------------------------------------------------------------------------
// Short rows: a wave takes P*RS consecutive rows and each slot a contiguous block of RS of
// them, so a slot's edges form one contiguous run that it walks as a single chunk stream
// (prefetching across row boundaries).  RS is kRowsPerWave / P, or 1 on graphs too small to
// give kFillWaves waves that many rows each (the grid then has one row per slot).  Rows with
// deg > short_max belong to the segment kernel and are skipped; short_max = INT_MAX without a
// plan.
constexpr int kRowsPerWave = 16;
constexpr int64_t kFillWaves = 2048;   // 256 CUs x 8 waves
// Slot width of the short-row kernel (lanes per row in flight).
constexpr int kShortSlotLanes = 32;

template <typename T, int H, int D, int MODE, class TAB, int GMAX, int RS>
__global__ __launch_bounds__(kBlock) void spmm_short_kernel(const int32_t* __restrict__ row_ptr,
                                                            const int32_t* __restrict__ col, int64_t n_rows,
                                                            int64_t n_src, const float* __restrict__ sc,
                                                            const T* __restrict__ qf, const T* __restrict__ kf,
                                                            const T* __restrict__ vf, float scale,
                                                            float* __restrict__ out, int short_max) {
    using E = Engine<T, H, D, MODE, TAB, GMAX>;
    constexpr int P = E::P, G = E::G, HD = E::HD, SC = E::SC, NV = E::NV, SM = E::SM, CM = E::CM;
    static_assert(RS + 1 <= G, "a slot holds its rows' row_ptr entries");
    const int lane = lane_id();
    const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    const int64_t wb = wave * P * RS;
    if (wb >= n_rows) return;
    __shared__ __align__(16) float stage[kWavesPerBlock * P * E::kStage];
    // each slot's output row, for the coalesced stores of 16-bit features
    constexpr bool kRowLds = E::EPP == 8;
    __shared__ __align__(16) float orow[kRowLds ? kWavesPerBlock * P * HD : 4];
    float* my_row = orow + (kRowLds ? (threadIdx.x / kWave * P + lane / G) * HD : 0);
    const TAB vt(vf, n_src);
    const TAB kt(MODE == kLayer ? kf : vf, n_src);
    E eng;
    eng.init_lane(lane, stage + (threadIdx.x / kWave * P + lane / G) * E::kStage);
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
    float s[SM];
    int cv[CM];
    eng.reset();
    eng.load_chunk(col, sc, e0, e1, s, cv);
    if constexpr (MODE == kLayer) {
        uint4 raw[NV];
        eng.load_q_raw(qf + (row0 + it) * HD, raw);
        eng.set_q(raw);
    }
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
        float s_n[SM] = {};
        int cv_n[CM] = {};
        uint4 qraw_n[NV] = {};   // the next row's query (kLayer): loaded whenever it is used
        if constexpr (MODE == kLayer) {
            const T* qn = (nit != it && nit < RS) ? qf + (row0 + nit) * HD : nullptr;
            eng.consume_layer(col, kt, vt, scale, c, e1, cv, nc, ne, cv_n, qn, qraw_n);
        } else {
            eng.consume_scores(col, sc, vt, c, e1, s, cv, nc, ne, s_n, cv_n);
        }
        if (nit != it) {
            eng.finish();
            if constexpr (kRowLds) eng.store_row_lds(out + (row0 + it) * HD, my_row, true);
            else eng.store_row(out + (row0 + it) * HD, true);
            if (nit >= RS) break;
            eng.reset();
            if constexpr (MODE == kLayer) eng.set_q(qraw_n);
            e1 = ne;
        }
        it = nit;
        c = nc;
#pragma unroll
        for (int k = 0; k < SM; ++k) s[k] = s_n[k];
#pragma unroll
        for (int k = 0; k < CM; ++k) cv[k] = cv_n[k];
    }
}

// ---------------------------------------------------------------------------------------------
// Long rows and hub segments: one 256-thread workgroup per segment of the plan's segment table
// (a grid of up to kSegmentGrid workgroups striding over the table; counts read on the device).  The
// 4*P slots split the segment's edges into contiguous sub-ranges, leave their states in LDS, and
// the workgroup merges them.  A long row (slot < 0) is written out; a hub segment's state goes to
// the plan's partial buffer.
template <typename T, int H, int D, int MODE, class TAB>
__global__ __launch_bounds__(kBlock) void spmm_segment_kernel(const int32_t* __restrict__ col, int64_t n_src,
                                                              const float* __restrict__ sc,
                                                              const T* __restrict__ qf, const T* __restrict__ kf,
                                                              const T* __restrict__ vf, float scale,
                                                              float* __restrict__ out, PlanView plan) {
    using E = Engine<T, H, D, MODE, TAB>;
    constexpr int NS = kWavesPerBlock * E::P;   // slots per workgroup
    constexpr int HD = E::HD;
    constexpr int SS = HD + 2 * H;              // floats per state
    __shared__ __align__(16) float lds[NS * SS];
    __shared__ __align__(16) float stage[NS * E::kStage];
    const TAB vt(vf, n_src);
    const TAB kt(MODE == kLayer ? kf : vf, n_src);
    const int lane = lane_id();
    const int gs = (threadIdx.x / kWave) * E::P + lane / E::G;
    const int n_segs = plan.counts[kNSegs];
    E eng;
    eng.init_lane(lane, stage + gs * E::kStage);
    for (int s = blockIdx.x; s < n_segs; s += gridDim.x) {
        const int4 sg = plan.segs[s];   // row, e_begin, e_end, slot
        const int64_t len = (int64_t)sg.z - sg.y;
        const int b = sg.y + (int)(len * gs / NS);
        const int e = sg.y + (int)(len * (gs + 1) / NS);
        eng.run_range(col, sc, qf + (int64_t)sg.x * HD, kt, vt, scale, b, e);
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
// Hub rows: merge the states of a row's segments and write the row.  One workgroup per hub row.
//  1. per-head max and sum: the 256 threads split the segments and merge (m, z) pairs, then an
//     xor-shuffle tree and a 4-wave merge through LDS give M[h], Z[h];
//  2. acc: thread groups split the segments (groups = 256 / (H*D) when H*D < 256), each thread
//     owning one element per group, with coalesced loads of the segments' acc rows and unrolled
//     loops; the groups' sums meet in LDS.
template <int MODE, int HMAX>
__global__ __launch_bounds__(kBlock) void spmm_hub_merge_kernel(float* __restrict__ out, int H, int D,
                                                                PlanView plan) {
    __shared__ float lm[kWavesPerBlock][HMAX], lz[kWavesPerBlock][HMAX];
    __shared__ float gM[HMAX], gZ[HMAX];
    __shared__ float part[kBlock];
    const int HD = H * D;
    const int t = threadIdx.x, lane = lane_id(), w = t / kWave;
    const int groups = HD < kBlock ? kBlock / HD : 1;
    const int g = HD < kBlock ? t / HD : 0;
    const int64_t sf = plan.state_floats;
    const int n_hubs = plan.counts[kNHubs];
    for (int hb = blockIdx.x; hb < n_hubs; hb += gridDim.x) {
        const int4 hr = plan.hubs[hb];   // row, first segment, n segments
        const float* p0 = plan.partials + (int64_t)hr.y * sf;
        if constexpr (MODE != kAgg) {
            float m[HMAX], z[HMAX];
#pragma unroll
            for (int h = 0; h < HMAX; ++h) {
                m[h] = -INFINITY;
                z[h] = 0.f;
            }
            for (int c = t; c < hr.z; c += kBlock) {
                const float* pc = p0 + (int64_t)c * sf;
#pragma unroll
                for (int h = 0; h < HMAX; ++h) {
                    if (h < H) {
                        const float mc = pc[h], zc = pc[H + h];
                        const float mn = fmaxf(m[h], mc);
                        z[h] = (m[h] == -INFINITY ? 0.f : z[h] * exp_fast(m[h] - mn)) +
                               (mc == -INFINITY ? 0.f : zc * exp_fast(mc - mn));
                        m[h] = mn;
                    }
                }
            }
#pragma unroll
            for (int h = 0; h < HMAX; ++h) {
                if (h < H) {
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
            }
            __syncthreads();
            if (t < H) {
                float M = -INFINITY, Z = 0.f;
#pragma unroll
                for (int i = 0; i < kWavesPerBlock; ++i) M = fmaxf(M, lm[i][t]);
#pragma unroll
                for (int i = 0; i < kWavesPerBlock; ++i)
                    if (lm[i][t] != -INFINITY) Z = fmaf(lz[i][t], exp_fast(lm[i][t] - M), Z);
                gM[t] = M;
                gZ[t] = Z;
            }
            __syncthreads();
        }
        for (int el0 = 0; el0 < HD; el0 += kBlock) {
            const int el = el0 + (HD < kBlock ? t % HD : t);
            const bool live = el < HD && g < groups;
            const int h = live ? el / D : 0;
            const float M = (MODE != kAgg) ? gM[h] : 0.f;
            float A = 0.f;
            if (live) {
#pragma unroll 8
                for (int c = g; c < hr.z; c += groups) {
                    const float* pc = p0 + (int64_t)c * sf;
                    const float wgt = (MODE != kAgg) ? (pc[h] == -INFINITY ? 0.f : exp_fast(pc[h] - M)) : 1.f;
                    A = fmaf(pc[2 * H + el], wgt, A);
                }
            }
            part[t] = A;
            __syncthreads();
            if (live && g == 0) {
                for (int i = 1; i < groups; ++i) A += part[i * HD + (t % HD)];
                out[(int64_t)hr.x * HD + el] = (MODE == kAgg) ? A : A / gZ[h];
            }
            __syncthreads();
        }
    }
}

template <int MODE>
hipError_t launch_spmm_mode(int dtype, int H, int D, const int32_t* row_ptr, const int32_t* col, int64_t n_rows,
                            int64_t n_src, const float* sc, const void* q, const void* k, const void* v, float scale,
                            float* out, const PlanView* plan, hipStream_t stream) {
    const bool ok = dispatch_shape(dtype, H, D, [&](auto tag) {
        using Tag = decltype(tag);
        using T = typename Tag::type;
        constexpr int HH = Tag::H, DD = Tag::D;
        constexpr int RB = Geo<T, HH, DD>::RB;
        const T* qt = static_cast<const T*>(q);
        const T* kt = static_cast<const T*>(k);
        const T* vt = static_cast<const T*>(v);
        // rows per slot: kRowsPerWave / P when that still gives kFillWaves waves, else 1
        constexpr int P = Geo<T, HH, DD, kShortSlotLanes>::P;
        constexpr int RS_MAX = kRowsPerWave / P;
        const bool small = n_rows < kFillWaves * kRowsPerWave;
        const int64_t rpw = small ? P : kRowsPerWave;
        const int64_t waves = (n_rows + rpw - 1) / rpw;
        const unsigned blocks = grid_for(waves, kWavesPerBlock, INT32_MAX);
        const int short_max = plan ? plan->short_max : INT32_MAX;
        auto go = [&](auto tab_tag) {
            using TAB = typename decltype(tab_tag)::type;
            if (plan)
                hipLaunchKernelGGL((spmm_segment_kernel<T, HH, DD, MODE, TAB>),
                                   dim3(grid_for(plan->seg_capacity, 1, kSegmentGrid)), dim3(kBlock), 0,
                                   stream, col, n_src, sc, qt, kt, vt, scale, out, *plan);
            if (small)
                hipLaunchKernelGGL((spmm_short_kernel<T, HH, DD, MODE, TAB, kShortSlotLanes, 1>), dim3(blocks),
                                   dim3(kBlock), 0, stream, row_ptr, col, n_rows, n_src, sc, qt, kt, vt, scale, out,
                                   short_max);
            else
                hipLaunchKernelGGL((spmm_short_kernel<T, HH, DD, MODE, TAB, kShortSlotLanes, RS_MAX>), dim3(blocks),
                                   dim3(kBlock), 0, stream, row_ptr, col, n_rows, n_src, sc, qt, kt, vt, scale, out,
                                   short_max);
        };
        // gathered tables below 4 GiB are read with 32-bit buffer offsets
        if (n_src * (int64_t)RB <= (int64_t)UINT32_MAX) go(TypeTag<Tab32<RB>>{});
        else go(TypeTag<Tab64<RB>>{});
    });
    if (!ok) return hipErrorInvalidValue;
    if (plan)
        hipLaunchKernelGGL((spmm_hub_merge_kernel<MODE, 16>), dim3(grid_for(plan->hub_capacity, 1, kPersistentBlocks)),
                           dim3(kBlock), 0, stream, out, H, D, *plan);
    return hipGetLastError();
}

}  // namespace gat
