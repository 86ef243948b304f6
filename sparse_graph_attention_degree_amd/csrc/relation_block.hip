// Dense relation-biased attention block (POPCORNBENCH l2_p4, the reference-model passage): per
// batch element, LayerNorm of the node rows, bias-free q/k/v projections, a per-pair bias from a
// Linear-SiLU-Linear MLP over pair features, masked multi-head softmax attention, the output
// projection and a residual on the raw nodes.  The page's shapes (4 x 24 nodes, 96 features, 4
// heads, 16 pair features) are far too small to fill the device, so the whole block for one batch
// element runs in one workgroup out of LDS -- one launch per call, no intermediate reaches HBM --
// and many batch elements run as many workgroups.
//
// LDS per workgroup (floats): xn / o [N*D], q, k, v [N*D] each, logits [H*N*N] (at most
// kRbMaxLds bytes; the C-ABI refuses larger shapes).  Steps, separated
// by workgroup barriers:
//  1. LayerNorm: a wave per node row, mean and variance by xor-shuffle sums over the row.
//  2. q, k, v: a thread per output column of each projection, rows in groups of 8 held in
//     registers while the weight row streams through (16-byte loads).
//  3. pair bias: a thread per (i, j) pair runs the MLP in registers (masked pairs get -inf).
//  4. logits: a thread per (h, i, j): scaled q.k over the head's columns plus the bias.
//  5. softmax: a thread per (h, i) row; a row with every pair masked becomes all zeros.
//  6. o = a v: a thread per (i, column).
//  7. out = x + o Wo^T: as step 2, with the residual added at the store.
#include <math.h>

#include "kernels.hpp"

namespace gat {

namespace {

constexpr int kRbRows = 8;   // node rows per register group in the projections

// y[i, r] = sum_c a[i, c] * w[r, c] for rows i < n, columns r < m (w row-major [m, kdim], global);
// a in LDS [n, kdim]; y in LDS [n, ldy] at column offset; thread per column.
__device__ void rb_project(const float* __restrict__ a, int n, int kdim, const float* __restrict__ w, int m,
                           float* y, int ldy) {
    for (int r = threadIdx.x; r < m; r += kBlock) {
        const float* wr = w + (int64_t)r * kdim;
        for (int i0 = 0; i0 < n; i0 += kRbRows) {
            float acc[kRbRows];
#pragma unroll
            for (int u = 0; u < kRbRows; ++u) acc[u] = 0.f;
            for (int c = 0; c < kdim; c += 4) {
                const float4 wv = *reinterpret_cast<const float4*>(wr + c);
#pragma unroll
                for (int u = 0; u < kRbRows; ++u) {
                    if (i0 + u < n) {
                        const float4 av = *reinterpret_cast<const float4*>(a + (i0 + u) * kdim + c);
                        acc[u] = fmaf(av.x, wv.x, fmaf(av.y, wv.y, fmaf(av.z, wv.z, fmaf(av.w, wv.w, acc[u]))));
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < kRbRows; ++u)
                if (i0 + u < n) y[(i0 + u) * ldy + r] = acc[u];
        }
    }
}

__global__ __launch_bounds__(kBlock) void relation_block_kernel(
    const float* nodes, const float* __restrict__ pair, const float* __restrict__ mask,
    const float* __restrict__ gamma, const float* __restrict__ beta, float eps, const float* __restrict__ wq,
    const float* __restrict__ wk, const float* __restrict__ wv, const float* __restrict__ wo,
    const float* __restrict__ w1, const float* __restrict__ b1,
    const float* __restrict__ w2, const float* __restrict__ b2, int N, int D, int H, int P,
    float* out) {
    extern __shared__ __align__(16) float lds[];
    const int b = blockIdx.x;
    const int t = threadIdx.x, lane = lane_id(), w = t / kWave;
    const int ND = N * D, hd = D / H;
    float* xn = lds;            // then o
    float* qs = lds + ND;
    float* ks = qs + ND;
    float* vs = ks + ND;
    float* lg = vs + ND;        // [H][N][N]
    const float* x = nodes + (int64_t)b * ND;

    // 1. LayerNorm
    for (int i = w; i < N; i += kWavesPerBlock) {
        float s = 0.f;
        for (int d = lane; d < D; d += kWave) s += x[i * D + d];
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) s += shfl_xor(s, o);
        const float mean = s / D;
        float v2 = 0.f;
        for (int d = lane; d < D; d += kWave) {
            const float c = x[i * D + d] - mean;
            v2 = fmaf(c, c, v2);
        }
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) v2 += shfl_xor(v2, o);
        const float rstd = 1.f / sqrtf(v2 / D + eps);
        for (int d = lane; d < D; d += kWave) xn[i * D + d] = (x[i * D + d] - mean) * rstd * gamma[d] + beta[d];
    }
    __syncthreads();

    // 2. q, k, v
    rb_project(xn, N, D, wq, D, qs, D);
    rb_project(xn, N, D, wk, D, ks, D);
    rb_project(xn, N, D, wv, D, vs, D);

    // 3. pair bias, straight into the logit buffer (masked pairs: -inf in every head)
    const float* pb = pair + (int64_t)b * N * N * P;
    const float* mb = mask + (int64_t)b * N * N;
    for (int pj = t; pj < N * N; pj += kBlock) {
        if (mb[pj] < 0.5f) {
            for (int h = 0; h < H; ++h) lg[h * N * N + pj] = -INFINITY;
            continue;
        }
        const float* f = pb + (int64_t)pj * P;
        float bias[kRbMaxHeads];
#pragma unroll
        for (int h = 0; h < kRbMaxHeads; ++h) bias[h] = h < H ? b2[h] : 0.f;
        for (int p = 0; p < P; ++p) {
            float hsum = b1[p];
            for (int c = 0; c < P; ++c) hsum = fmaf(w1[p * P + c], f[c], hsum);
            const float hid = hsum / (1.f + exp_fast(-hsum));
#pragma unroll
            for (int h = 0; h < kRbMaxHeads; ++h)
                if (h < H) bias[h] = fmaf(w2[h * P + p], hid, bias[h]);
        }
#pragma unroll
        for (int h = 0; h < kRbMaxHeads; ++h)
            if (h < H) lg[h * N * N + pj] = bias[h];
    }
    __syncthreads();

    // 4. logits
    const float scale = 1.f / sqrtf((float)hd);
    for (int e = t; e < H * N * N; e += kBlock) {
        if (lg[e] == -INFINITY) continue;
        const int h = e / (N * N), i = (e / N) % N, j = e % N;
        const float* qi = qs + i * D + h * hd;
        const float* kj = ks + j * D + h * hd;
        float d = 0.f;
        for (int c = 0; c < hd; ++c) d = fmaf(qi[c], kj[c], d);
        lg[e] = fmaf(d, scale, lg[e]);
    }
    __syncthreads();

    // 5. softmax per (h, i); a row with every pair masked is all zeros
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

    // 6. o = a v (over xn, no longer needed)
    float* o = xn;
    for (int e = t; e < ND; e += kBlock) {
        const int i = e / D, c = e % D, h = c / hd;
        const float* a = lg + (h * N + i) * N;
        float s = 0.f;
        for (int j = 0; j < N; ++j) s = fmaf(a[j], vs[j * D + c], s);
        o[e] = s;
    }
    __syncthreads();

    // 7. out = x + o Wo^T  (projected into q's buffer, then the residual at the store)
    rb_project(o, N, D, wo, D, qs, D);
    __syncthreads();
    float* ob = out + (int64_t)b * ND;
    for (int e = t; e < ND; e += kBlock) ob[e] = x[e] + qs[e];
}

}  // namespace

size_t relation_block_lds_bytes(int N, int D, int H) { return ((size_t)4 * N * D + (size_t)H * N * N) * 4; }

hipError_t launch_relation_block(const float* nodes, const float* pair, const float* mask, const float* gamma,
                                 const float* beta, float eps, const float* wq, const float* wk, const float* wv,
                                 const float* wo, const float* w1, const float* b1, const float* w2, const float* b2,
                                 int64_t B, int N, int D, int H, int P, float* out, hipStream_t stream) {
    if (B == 0 || N == 0) return hipSuccess;
    const size_t lds = relation_block_lds_bytes(N, D, H);
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
