// Dense relation-biased attention block (POPCORNBENCH l2_p4, the reference-model passage): per
// batch element, LayerNorm of the node rows, bias-free q/k/v projections, a per-pair bias from a
// Linear-SiLU-Linear MLP over pair features, masked multi-head softmax attention, the output
// projection and a residual on the raw nodes.  The page's shapes (4 x 24 nodes, 96 features, 4
// heads, 16 pair features) are far too small to fill the device, so the whole block for one batch
// element runs in one workgroup out of LDS -- one launch per call, no intermediate reaches HBM --
// and many batch elements run as many workgroups.
//
// The block for one element is a chain of short dependent steps, so the design is about memory
// latency: every small input goes to LDS in one burst at the start, and the weight matrices stream
// through LDS in double-buffered blocks.  LDS per workgroup (floats): x / LayerNorm(x) / o [N*D],
// q, k, v [N*(D+1)] each, logits [H*N*N], the mask [N*N], the pair MLP's weights, and two blocks of
// weight rows (at most kRbMaxLds bytes; the C-ABI refuses larger shapes).  Steps, separated by
// workgroup barriers:
//  0. x, the mask and the MLP weights into LDS (all loads in flight together).
//  1. pair bias: the pair features stream through LDS (coalesced) in rounds; a thread per (i, j)
//     pair runs the MLP out of LDS, its SiLU outputs beside its features (masked pairs get -inf).
//  2. LayerNorm in place: a wave per node row, mean and variance by xor-shuffle sums over the row.
//  3. q, k, v: weight rows through LDS kRbCols at a time (coalesced 16-byte loads of the next block
//     issued before the current one is used); a thread per output.
//  4. logits: a thread per (h, i, j): scaled q.k over the head's columns plus the bias.
//  5. softmax: a thread per (h, i) row; a row with every pair masked becomes all zeros.
//  6. o = a v: a thread per (i, column).
//  7. out = x + o Wo^T: as step 2, with the residual (x re-read, L2-resident) added at the store.
#include <math.h>

#include <type_traits>

#include "kernels.hpp"

namespace gat {

namespace {

constexpr int kRbCols = 16;   // weight rows (output columns) staged in LDS per step

// LDS regions in floats, each starting on a 16-byte boundary
struct RbLayout {
    int xn, qs, ks, vs, lg, mk, mw, wbuf, total;
};

__host__ __device__ inline RbLayout rb_layout(int N, int D, int H, int P) {
    auto up = [](int v) { return (v + 3) & ~3; };
    RbLayout L{};
    int o = 0;
    L.xn = o, o += up(N * D);
    L.qs = o, o += up(N * (D + 1) > 2 * P + 1 ? N * (D + 1) : 2 * P + 1);   // also the pair-feature stage
    L.ks = o, o += up(N * (D + 1));
    L.vs = o, o += up(N * (D + 1));
    L.lg = o, o += up(H * N * N);
    L.mk = o, o += up(N * N);
    L.mw = o, o += up(P * P + P + H * P + H);
    L.wbuf = o, o += 2 * kRbCols * (D + 4);
    L.total = o;
    return L;
}

// y[i, r] = sum_c a[i, c] * w[r, c] for rows i < n and columns r < m.  w is row-major [m, kdim] in
// global memory (the same for every workgroup, so L2-resident); a is LDS [n, kdim] (16-byte rows).
// The weight rows go through LDS kRbCols at a time, double-buffered: the coalesced loads of the
// next block are issued before the current one is used, so one memory latency overlaps one block
// of arithmetic.  wbuf: 2 * kRbCols * (kdim + 4) floats (rows padded against bank conflicts).
__device__ void rb_project(const float* __restrict__ a, int n, int kdim, const float* __restrict__ w, int m,
                           float* y, int ldy, float* wbuf) {
    const int ldw = kdim + 4;
    const int nblk = (m + kRbCols - 1) / kRbCols;
    const int per = kRbCols * kdim / 4;   // float4s per block
    float4 pre[4];                         // this thread's share of the next block (<= 4 float4s)
    auto fetch = [&](int blk) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = threadIdx.x + u * kBlock;
            pre[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            const int r = blk * kRbCols + (4 * e) / kdim;
            if (e < per && r < m) pre[u] = *reinterpret_cast<const float4*>(w + (int64_t)r * kdim + (4 * e) % kdim);
        }
    };
    auto stash = [&](float* dst) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = threadIdx.x + u * kBlock;
            if (e < per) *reinterpret_cast<float4*>(dst + ((4 * e) / kdim) * ldw + (4 * e) % kdim) = pre[u];
        }
    };
    fetch(0);
    for (int blk = 0; blk < nblk; ++blk) {
        float* cur = wbuf + (blk & 1) * kRbCols * ldw;
        stash(cur);
        __syncthreads();
        if (blk + 1 < nblk) fetch(blk + 1);
        for (int o = threadIdx.x; o < n * kRbCols; o += kBlock) {
            const int i = o / kRbCols, rr = o % kRbCols, r = blk * kRbCols + rr;
            if (r >= m) continue;
            const float* ar = a + i * kdim;
            const float* wr = cur + rr * ldw;
            float acc = 0.f;
#pragma unroll 8
            for (int c = 0; c < kdim; c += 4) {
                const float4 av = *reinterpret_cast<const float4*>(ar + c);
                const float4 wv = *reinterpret_cast<const float4*>(wr + c);
                acc = fmaf(av.x, wv.x, fmaf(av.y, wv.y, fmaf(av.z, wv.z, fmaf(av.w, wv.w, acc))));
            }
            y[i * ldy + r] = acc;
        }
    }
    __syncthreads();
}

// LayerNorm of rows [0, N) of xn [N][D] in place: a wave per row.
__device__ void rb_layernorm(float* xn, int N, int D, const float* __restrict__ gamma,
                             const float* __restrict__ beta, float eps) {
    const int lane = lane_id(), w = threadIdx.x / kWave;
    for (int i = w; i < N; i += kWavesPerBlock) {
        float s = 0.f;
        for (int d = lane; d < D; d += kWave) s += xn[i * D + d];
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) s += shfl_xor(s, o);
        const float mean = s / D;
        float v2 = 0.f;
        for (int d = lane; d < D; d += kWave) {
            const float c = xn[i * D + d] - mean;
            v2 = fmaf(c, c, v2);
        }
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) v2 += shfl_xor(v2, o);
        const float rstd = 1.f / sqrtf(v2 / D + eps);
        for (int d = lane; d < D; d += kWave) xn[i * D + d] = (xn[i * D + d] - mean) * rstd * gamma[d] + beta[d];
    }
}

// Steps 4-6 on q, k, v [N][ld] and the biased logits lg [H][N][N] (-inf where masked): scaled q.k
// added to the bias (lanes along j: k rows padded to ld = D + 1 land in different banks), the
// softmax per (h, i) (a row with every pair masked becomes all zeros), and o = a v into o [N][D].
__device__ void rb_attend(const float* qs, const float* ks, const float* vs, int ld, int ldv, float* lg, int N,
                          int D, int H, float* o) {
    const int t = threadIdx.x, hd = D / H;
    const float scale = 1.f / sqrtf((float)hd);
    for (int e = t; e < H * N * N; e += kBlock) {
        if (lg[e] == -INFINITY) continue;
        const int h = e / (N * N), i = (e / N) % N, j = e % N;
        const float* qi = qs + i * ld + h * hd;
        const float* kj = ks + j * ld + h * hd;
        float d = 0.f;
#pragma unroll 8
        for (int c = 0; c < hd; ++c) d = fmaf(qi[c], kj[c], d);
        lg[e] = fmaf(d, scale, lg[e]);
    }
    __syncthreads();
    for (int hi = t; hi < H * N; hi += kBlock) {
        float* row = lg + hi * N;
        float m = -INFINITY;
        for (int j = 0; j < N; ++j) m = fmaxf(m, row[j]);
        if (m == -INFINITY) {
            for (int j = 0; j < N; ++j) row[j] = 0.f;
            continue;
        }
        float z = 0.f;
        for (int j = 0; j < N; ++j) {
            const float p = row[j] == -INFINITY ? 0.f : exp_fast(row[j] - m);
            row[j] = p;
            z += p;
        }
        const float rz = 1.f / z;
        for (int j = 0; j < N; ++j) row[j] *= rz;
    }
    __syncthreads();
    for (int e = t; e < N * D; e += kBlock) {
        const int i = e / D, c = e % D, h = c / hd;
        const float* a = lg + (h * N + i) * N;
        float s = 0.f;
#pragma unroll 8
        for (int j = 0; j < N; ++j) s = fmaf(a[j], vs[j * ldv + c], s);
        o[e] = s;
    }
    __syncthreads();
}

__global__ __launch_bounds__(kBlock) void relation_block_kernel(
    const float* nodes, const float* __restrict__ pair, const float* __restrict__ mask,
    const float* __restrict__ gamma, const float* __restrict__ beta, float eps, const float* __restrict__ wq,
    const float* __restrict__ wk, const float* __restrict__ wv, const float* __restrict__ wo,
    const float* __restrict__ w1, const float* __restrict__ b1, const float* __restrict__ w2,
    const float* __restrict__ b2, int N, int D, int H, int P, float* out) {
    extern __shared__ __align__(16) float lds[];
    const int b = blockIdx.x;
    const int t = threadIdx.x, lane = lane_id(), w = t / kWave;
    const int ND = N * D, ld = D + 1;   // q/k/v rows padded by one float (bank spread)
    const RbLayout L = rb_layout(N, D, H, P);
    float* xn = lds + L.xn;          // [N][D]: x, then LayerNorm(x), then o
    float* qs = lds + L.qs;          // [N][ld]
    float* ks = lds + L.ks;
    float* vs = lds + L.vs;
    float* lg = lds + L.lg;          // [H][N][N]
    float* mk = lds + L.mk;          // [N][N]
    float* mw = lds + L.mw;          // pair MLP: w1 [P*P], b1 [P], w2 [H*P], b2 [H]
    float* wbuf = lds + L.wbuf;      // two blocks of kRbCols weight rows
    const float* x = nodes + (int64_t)b * ND;

    // 0. everything small into LDS with all loads in flight together: x, the mask, the MLP weights
    for (int e = t; e < ND / 4; e += kBlock)
        reinterpret_cast<float4*>(xn)[e] = reinterpret_cast<const float4*>(x)[e];
    const float* mb = mask + (int64_t)b * N * N;
    for (int e = t; e < N * N; e += kBlock) mk[e] = mb[e];
    for (int e = t; e < P * P; e += kBlock) mw[e] = w1[e];
    for (int e = t; e < P; e += kBlock) mw[P * P + e] = b1[e];
    for (int e = t; e < H * P; e += kBlock) mw[P * P + P + e] = w2[e];
    for (int e = t; e < H; e += kBlock) mw[P * P + P + H * P + e] = b2[e];
    __syncthreads();

    // 1. pair bias, straight into the logit buffer (masked pairs: -inf in every head).  Rounds of
    //    R pairs: their features (contiguous) staged with coalesced loads in the q/k/v region, which
    //    is free until step 3; then a thread per pair runs the MLP with the hidden layer in registers.
    {
        const float* pb = pair + (int64_t)b * N * N * P;
        const float* W1 = mw;
        const float* B1 = mw + P * P;
        const float* W2 = B1 + P;
        const float* B2 = W2 + H * P;
        float* fs = qs;                                      // [R][2P + 1]: features, then SiLU outputs
        const int rl = 2 * P + 1;
        const int cap = (L.lg - L.qs) / rl;                  // >= 1 by the layout
        const int R = cap < kBlock ? cap : kBlock;
        for (int p0 = 0; p0 < N * N; p0 += R) {
            const int cnt = (N * N - p0) < R ? (N * N - p0) : R;
            for (int e = t; e < cnt * P; e += kBlock) fs[(e / P) * rl + e % P] = pb[(int64_t)p0 * P + e];
            __syncthreads();
            const int pj = p0 + t;
            if (t < cnt) {
                if (mk[pj] < 0.5f) {
                    for (int h = 0; h < H; ++h) lg[h * N * N + pj] = -INFINITY;
                } else {
                    float* row = fs + t * rl;
                    for (int p = 0; p < P; ++p) {
                        const float* w1r = W1 + p * P;
                        float hs = B1[p];
#pragma unroll 8
                        for (int c = 0; c < P; ++c) hs = fmaf(w1r[c], row[c], hs);
                        row[P + p] = hs / (1.f + exp_fast(-hs));
                    }
                    for (int h = 0; h < H; ++h) {
                        const float* w2r = W2 + h * P;
                        float bs = B2[h];
#pragma unroll 8
                        for (int p = 0; p < P; ++p) bs = fmaf(w2r[p], row[P + p], bs);
                        lg[h * N * N + pj] = bs;
                    }
                }
            }
            __syncthreads();
        }
    }

    // 2. LayerNorm in place
    rb_layernorm(xn, N, D, gamma, beta, eps);
    __syncthreads();

    // 3. q, k, v
    rb_project(xn, N, D, wq, D, qs, ld, wbuf);
    rb_project(xn, N, D, wk, D, ks, ld, wbuf);
    rb_project(xn, N, D, wv, D, vs, ld, wbuf);

    // 4-6. logits, softmax, o = a v (over xn, no longer needed)
    float* o = xn;
    rb_attend(qs, ks, vs, ld, ld, lg, N, D, H, o);

    // 7. out = x + o Wo^T  (projected into q's buffer, then the residual at the store)
    rb_project(o, N, D, wo, D, qs, ld, wbuf);
    float* ob = out + (int64_t)b * ND;
    for (int e = t; e < ND; e += kBlock) ob[e] = x[e] + qs[(e / D) * ld + e % D];
}

// ------------------------------------------------------------------ matrix-core path
// For pair_dim 16, dim a multiple of 16 (at most 128) and up to 64 nodes, the dense products run on
// v_mfma_f32_16x16x4f32 (fp32 in, fp32 sums; 64 MACs per lane per instruction against one FMA):
// the four dim x dim projections and both layers of the pair MLP.  Lane l of a 16x16x4 step
// supplies A[l % 16][l / 16] and B[l / 16][l % 16]; accumulator register r of lane l is
// C[4 (l / 16) + r][l % 16].  A lane reads four consecutive k of its A row and of its B column as
// one 16-byte load and feeds them to four steps, so step s sums k = 4 (l / 16) + s of each 16-k
// block: every k still meets its own partner once.
//  - projections y = a w^T: A = rows of a (LDS, rows past N zero), B = rows of w (global, shared by
//    every workgroup, so L2-resident); each wave owns 16x16 output tiles, two at a time.
//  - pair MLP, per 16 pairs: layer 1 as h^T = W1 f^T (A = W1 rows, B = the pairs' features
//    straight from global), so lane l ends with hidden units 4 (l / 16) + r of pair l % 16, which
//    after + b1 and SiLU are exactly the B operand of layer 2, bias^T = W2 silu(h)^T, step s = r.
// The logits, softmax and o = a v stay on the vector units (about a tenth of the products).
typedef float rb_f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRbFastP = 16;
constexpr int kRbFastMaxN = 64;
constexpr int kRbPairBatch = 8;   // pair tiles whose features a wave loads at once

__device__ __forceinline__ rb_f32x4 rb_mfma(float a, float b, rb_f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// LDS of the matrix-core kernel (floats): three row arrays and the logits, 37 KB at the page's shape,
// so four workgroups share a CU.  xn [N][D] holds x, then LayerNorm(x), then v; qs [N][D+1] holds q,
// then o (row pitch D); ks [N][D+1] holds k, then o Wo^T.
struct RbFastLayout {
    int xn, qs, ks, lg, mb, total;
};

__host__ __device__ inline RbFastLayout rb_fast_layout(int N, int D, int H) {
    auto up = [](int v) { return (v + 3) & ~3; };
    RbFastLayout L{};
    int o = 0;
    L.xn = o, o += up(N * D);
    L.qs = o, o += up(N * (D + 1));
    L.ks = o, o += up(N * (D + 1));
    L.lg = o, o += up(H * N * N);
    L.mb = o, o += up(kRbFastP + H);            // b1, b2
    L.total = o;
    return L;
}

// One 16x16 tile of y = a w^T over KB blocks of 16 k (k past D reads 0).
// One 16x16 tile of y = a w^T over KB blocks of 16 k: a [N][lda] in LDS, w [D][D] in global memory;
// k past D and rows past N read 0.  The w fragments of a tile are loaded first (one L2 round trip),
// the a fragments from LDS as each block is reached.
template <int KB>
__device__ __forceinline__ void rb_tile_wload(const float* __restrict__ w, int D, int ct, float4 (&wv)[KB]) {
    const int lane = lane_id(), li = lane % 16, lk = 4 * (lane / 16);
    const float* wr = w + (int64_t)(ct * 16 + li) * D + lk;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
        wv[kb] = 16 * kb + lk < D ? *reinterpret_cast<const float4*>(wr + 16 * kb) : make_float4(0.f, 0.f, 0.f, 0.f);
}

template <int KB>
__device__ __forceinline__ rb_f32x4 rb_tile_mfma(const float* a, int lda, int N, int D, int rt,
                                                 const float4 (&wv)[KB]) {
    const int lane = lane_id(), li = lane % 16, lk = 4 * (lane / 16);
    const int row = rt * 16 + li;
    const float* ar = a + row * lda + lk;
    rb_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const float4 av = row < N && 16 * kb + lk < D ? *reinterpret_cast<const float4*>(ar + 16 * kb)
                                                      : make_float4(0.f, 0.f, 0.f, 0.f);
        acc = rb_mfma(av.x, wv[kb].x, acc);
        acc = rb_mfma(av.y, wv[kb].y, acc);
        acc = rb_mfma(av.z, wv[kb].z, acc);
        acc = rb_mfma(av.w, wv[kb].w, acc);
    }
    return acc;
}

__device__ __forceinline__ void rb_tile_store(rb_f32x4 acc, int rt, int ct, int N, float* y, int ldy) {
    const int lane = lane_id(), li = lane % 16, lk = 4 * (lane / 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = rt * 16 + lk + r;
        if (i < N) y[i * ldy + ct * 16 + li] = acc[r];
    }
}

// y[i, j] = sum_k a[i, k] w[j, k], i < N, j < D: a LDS [N][lda], w global [D][D] (row-major,
// [out, in]), y LDS with row pitch ldy (y must not overlap a).  A wave takes tiles wave, wave + 4, ...
// two at a time, with both tiles' w loads issued before the first MFMA.
template <int KB>
__device__ void rb_mfma_project(const float* a, int lda, const float* __restrict__ w, int N, int D, float* y,
                                int ldy) {
    const int wave = threadIdx.x / kWave;
    const int RT = (N + 15) / 16, CT = D / 16, T = RT * CT;
    for (int t0 = wave; t0 < T; t0 += 2 * kWavesPerBlock) {
        const int t1 = t0 + kWavesPerBlock;
        float4 wv0[KB], wv1[KB];
        rb_tile_wload<KB>(w, D, t0 % CT, wv0);
        if (t1 < T) rb_tile_wload<KB>(w, D, t1 % CT, wv1);
        rb_tile_store(rb_tile_mfma<KB>(a, lda, N, D, t0 / CT, wv0), t0 / CT, t0 % CT, N, y, ldy);
        if (t1 < T) rb_tile_store(rb_tile_mfma<KB>(a, lda, N, D, t1 / CT, wv1), t1 / CT, t1 % CT, N, y, ldy);
    }
}

// The same product written over a itself (y = a, row pitch lda): every tile is computed into
// registers first, then after a workgroup barrier -- every wave's reads of a done -- written.  All
// threads must call it.
template <int KB>
__device__ void rb_mfma_project_in_place(float* a, int lda, const float* __restrict__ w, int N, int D) {
    // at most (kRbFastMaxN / 16) row tiles x KB column tiles over the four waves
    constexpr int kRbMaxTilesPerWave = (kRbFastMaxN / 16) * KB / kWavesPerBlock;
    const int wave = threadIdx.x / kWave;
    const int RT = (N + 15) / 16, CT = D / 16, T = RT * CT;
    rb_f32x4 acc[kRbMaxTilesPerWave];
#pragma unroll
    for (int u = 0; u < kRbMaxTilesPerWave; u += 2) {
        const int t0 = wave + u * kWavesPerBlock, t1 = t0 + kWavesPerBlock;
        if (t0 >= T) break;
        float4 wv0[KB], wv1[KB];
        rb_tile_wload<KB>(w, D, t0 % CT, wv0);
        if (t1 < T) rb_tile_wload<KB>(w, D, t1 % CT, wv1);
        acc[u] = rb_tile_mfma<KB>(a, lda, N, D, t0 / CT, wv0);
        if (t1 < T) acc[u + 1] = rb_tile_mfma<KB>(a, lda, N, D, t1 / CT, wv1);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kRbMaxTilesPerWave; ++u) {
        const int tt = wave + u * kWavesPerBlock;
        if (tt >= T) break;
        rb_tile_store(acc[u], tt / CT, tt % CT, N, a, lda);
    }
}

template <int KB>
__global__ __launch_bounds__(kBlock, 4) void relation_block_mfma_kernel(
    const float* nodes, const float* __restrict__ pair, const float* __restrict__ mask,
    const float* __restrict__ gamma, const float* __restrict__ beta, float eps, const float* __restrict__ wq,
    const float* __restrict__ wk, const float* __restrict__ wv, const float* __restrict__ wo,
    const float* __restrict__ w1, const float* __restrict__ b1, const float* __restrict__ w2,
    const float* __restrict__ b2, int N, int D, int H, float* out) {
    extern __shared__ __align__(16) float lds[];
    const int b = blockIdx.x;
    const int t = threadIdx.x, lane = lane_id(), wave = t / kWave;
    const int li = lane % 16, lk = 4 * (lane / 16);
    const int ND = N * D, NN = N * N, ld = D + 1;
    const RbFastLayout L = rb_fast_layout(N, D, H);
    float* xn = lds + L.xn;          // [N][D]: x, LayerNorm(x), then v
    float* qs = lds + L.qs;          // [N][ld]: q, then o (pitch D)
    float* ks = lds + L.ks;          // [N][ld]: k, then o Wo^T
    float* lg = lds + L.lg;          // [H][N][N]
    float* mb = lds + L.mb;          // b1 [16], b2 [H]
    const float* x = nodes + (int64_t)b * ND;

    // 0. x and the MLP biases into LDS
    for (int e = t; e < ND / 4; e += kBlock)
        reinterpret_cast<float4*>(xn)[e] = reinterpret_cast<const float4*>(x)[e];
    if (t < kRbFastP) mb[t] = b1[t];
    if (t < H) mb[kRbFastP + t] = b2[t];
    __syncthreads();

    // 1. pair bias into the logit buffer (-inf where masked), 16 pairs per wave step
    {
        const float4 w1f = *reinterpret_cast<const float4*>(w1 + li * kRbFastP + lk);
        const float4 w2f = li < H ? *reinterpret_cast<const float4*>(w2 + li * kRbFastP + lk)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
        const float* fp = pair + (int64_t)b * NN * kRbFastP;
        const float* mg = mask + (int64_t)b * NN;
        const int PT = (NN + 15) / 16;
        // pairs pt*16 .. +15 with the features f of pair pt*16 + li (k = lk .. lk + 3) and its mask
        auto tile = [&](int pt, const float4& f, float keepv) {
            const int p = pt * 16 + li;
            rb_f32x4 h = {0.f, 0.f, 0.f, 0.f};
            h = rb_mfma(w1f.x, f.x, h);
            h = rb_mfma(w1f.y, f.y, h);
            h = rb_mfma(w1f.z, f.z, h);
            h = rb_mfma(w1f.w, f.w, h);
            float sl[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float hs = h[r] + mb[lk + r];
                sl[r] = hs / (1.f + exp_fast(-hs));
            }
            rb_f32x4 c = {0.f, 0.f, 0.f, 0.f};
            c = rb_mfma(w2f.x, sl[0], c);
            c = rb_mfma(w2f.y, sl[1], c);
            c = rb_mfma(w2f.z, sl[2], c);
            c = rb_mfma(w2f.w, sl[3], c);
            if (p < NN) {
                const bool keep = keepv >= 0.5f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int h2 = lk + r;
                    if (h2 < H) lg[h2 * NN + p] = keep ? c[r] + mb[kRbFastP + h2] : -INFINITY;
                }
            }
        };
        // the features and mask entries of kRbPairBatch tiles are loaded together, then consumed: one
        // memory latency per batch instead of one per tile
        for (int pt0 = wave; pt0 < PT; pt0 += kRbPairBatch * kWavesPerBlock) {
            float4 fb[kRbPairBatch];
            float kb[kRbPairBatch];
#pragma unroll
            for (int u = 0; u < kRbPairBatch; ++u) {
                const int p = (pt0 + u * kWavesPerBlock) * 16 + li;
                fb[u] = p < NN ? *reinterpret_cast<const float4*>(fp + (int64_t)p * kRbFastP + lk)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
                kb[u] = p < NN ? mg[p] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < kRbPairBatch; ++u)
                if (pt0 + u * kWavesPerBlock < PT) tile(pt0 + u * kWavesPerBlock, fb[u], kb[u]);
        }
    }

    // 2. LayerNorm in place
    rb_layernorm(xn, N, D, gamma, beta, eps);
    __syncthreads();

    // 3. q, k into their buffers, then v over LayerNorm(x) (all reads of xn before the writes)
    rb_mfma_project<KB>(xn, D, wq, N, D, qs, ld);
    rb_mfma_project<KB>(xn, D, wk, N, D, ks, ld);
    rb_mfma_project_in_place<KB>(xn, D, wv, N, D);
    __syncthreads();

    // 4-6. logits, softmax, o = a v into q's buffer (q is no longer read once the logits exist)
    rb_attend(qs, ks, xn, ld, D, lg, N, D, H, qs);

    // 7. out = x + o Wo^T (projected into k's buffer, then the residual at the store)
    rb_mfma_project<KB>(qs, D, wo, N, D, ks, ld);
    __syncthreads();
    float* ob = out + (int64_t)b * ND;
    for (int e = t; e < ND; e += kBlock) ob[e] = x[e] + ks[(e / D) * ld + e % D];
}

}  // namespace

size_t relation_block_lds_bytes(int N, int D, int H, int P) { return (size_t)rb_layout(N, D, H, P).total * 4; }

namespace {

template <int KB>
hipError_t launch_rb_fast(const float* nodes, const float* pair, const float* mask, const float* gamma,
                          const float* beta, float eps, const float* wq, const float* wk, const float* wv,
                          const float* wo, const float* w1, const float* b1, const float* w2, const float* b2,
                          int64_t B, int N, int D, int H, float* out, hipStream_t stream) {
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(relation_block_mfma_kernel<KB>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, kRbMaxLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const size_t lds = (size_t)rb_fast_layout(N, D, H).total * 4;
    hipLaunchKernelGGL(relation_block_mfma_kernel<KB>, dim3((unsigned)B), dim3(kBlock), lds, stream, nodes, pair,
                       mask, gamma, beta, eps, wq, wk, wv, wo, w1, b1, w2, b2, N, D, H, out);
    return hipGetLastError();
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

}  // namespace

hipError_t launch_relation_block(const float* nodes, const float* pair, const float* mask, const float* gamma,
                                 const float* beta, float eps, const float* wq, const float* wk, const float* wv,
                                 const float* wo, const float* w1, const float* b1, const float* w2, const float* b2,
                                 int64_t B, int N, int D, int H, int P, float* out, hipStream_t stream) {
    if (B == 0 || N == 0) return hipSuccess;
    // the matrix-core kernel where its shape conditions hold (16-byte operand loads included)
    if (P == kRbFastP && D % 16 == 0 && D <= 128 && N <= kRbFastMaxN && aligned16(pair) && aligned16(w1) &&
        aligned16(w2) && (size_t)rb_fast_layout(N, D, H).total * 4 <= kRbMaxLds) {
        auto go = [&](auto kb) {
            return launch_rb_fast<decltype(kb)::value>(nodes, pair, mask, gamma, beta, eps, wq, wk, wv, wo, w1, b1,
                                                       w2, b2, B, N, D, H, out, stream);
        };
        if (D <= 32) return go(std::integral_constant<int, 2>{});
        if (D <= 64) return go(std::integral_constant<int, 4>{});
        if (D <= 96) return go(std::integral_constant<int, 6>{});
        return go(std::integral_constant<int, 8>{});
    }
    const size_t lds = relation_block_lds_bytes(N, D, H, P);
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(relation_block_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, kRbMaxLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(relation_block_kernel, dim3((unsigned)B), dim3(kBlock), lds, stream, nodes, pair, mask,
                       gamma, beta, eps, wq, wk, wv, wo, w1, b1, w2, b2, N, D, H, P, out);
    return hipGetLastError();
}

}  // namespace gat
