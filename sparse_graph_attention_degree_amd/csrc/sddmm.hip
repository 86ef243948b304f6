// SDDMM over an edge list (POPCORNBENCH l1_p10, the reference model: gather
// src_feat[src_idx] and dst_feat[dst_idx], multiply, sum over the feature dim),
// extended to heads:  out[e,h] = scale * <dst_feat[dst_idx[e],h,:], src_feat[src_idx[e],h,:]>.
//
// The page's final design is a 32-lane group per edge with a lane-strided loop
// over the 128 features and a shuffle tree.  Here a slot of G lanes (common.hpp)
// owns one edge and each lane takes 16-byte pieces of both rows, so one wave64
// holds P edges per step and U steps of gathers are issued before any is used.
// The per-head sum over the LPH lanes of a head stays in registers (DPP, group_sum).  The waves
// sweep the edge list together (grid-stride), so with edges sorted by destination
// neighbouring waves share destination rows and output lines in L2; keeping the
// destination row in registers across repeated destinations, prefetching the next
// indices, and buffer loads each measured slower here and are not used.
#include "kernels.hpp"

namespace gat {

namespace {

template <typename T, int H, int D>
__global__ __launch_bounds__(kBlock) void sddmm_kernel(const int32_t* __restrict__ src_idx,
                                                       const int32_t* __restrict__ dst_idx, int64_t n_edges,
                                                       const T* __restrict__ sf, const T* __restrict__ df,
                                                       float scale, float* __restrict__ out) {
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
        int si = 0, di = 0;
        if (lane < EPI && base + lane < n_edges) {
            si = src_idx[base + lane];
            di = dst_idx[base + lane];
        }
        uint4 a[U][NV], b[U][NV];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int el = u * P + g;
            const int s_i = shfl(si, el), d_i = shfl(di, el);
            const bool valid = base + el < n_edges;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                if (valid) {
                    a[u][v] = ld16(df + (int64_t)d_i * HD + off[v]);
                    b[u][v] = ld16(sf + (int64_t)s_i * HD + off[v]);
                } else {
                    a[u][v] = make_uint4(0u, 0u, 0u, 0u);
                    b[u][v] = make_uint4(0u, 0u, 0u, 0u);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e = base + u * P + g;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                float fa[EPP], fb[EPP];
                unpack<T>(a[u][v], fa);
                unpack<T>(b[u][v], fb);
                float d = 0.f;
#pragma unroll
                for (int k = 0; k < EPP; ++k) d = fmaf(fa[k], fb[k], d);
                d = group_sum<LPH>(d);
                if (e < n_edges && (v * G + q) % LPH == 0) out[e * H + hv[v]] = scale * d;
            }
        }
    }
}

}  // namespace

hipError_t launch_sddmm(int dtype, int H, int D, const int32_t* src_idx, const int32_t* dst_idx, int64_t n_edges,
                        const void* src_feat, int64_t /*n_src*/, const void* dst_feat, int64_t /*n_dst*/,
                        float scale, float* out, hipStream_t stream) {
    if (n_edges == 0) return hipSuccess;
    const bool ok = dispatch_shape(dtype, H, D, [&](auto tag) {
        using Tag = decltype(tag);
        using T = typename Tag::type;
        using Gm = Geo<T, Tag::H, Tag::D>;
        constexpr int UMAX = (8 / Gm::NV) > 1 ? (8 / Gm::NV) : 1;
        constexpr int U = UMAX * Gm::P <= kWave ? UMAX : kWave / Gm::P;
        const int64_t waves = (n_edges + U * Gm::P - 1) / (U * Gm::P);
        hipLaunchKernelGGL((sddmm_kernel<T, Tag::H, Tag::D>), dim3(grid_for(waves, kWavesPerBlock, edge_grid_cap())),
                           dim3(kBlock), 0, stream, src_idx, dst_idx, n_edges, static_cast<const T*>(src_feat),
                           static_cast<const T*>(dst_feat), scale, out);
    });
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gat
