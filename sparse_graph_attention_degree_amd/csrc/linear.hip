// Node projections (the nn.Linear steps on either side of the attention in the l2_p4 reference
// model): y[m, n] = bias[n] + sum_k x[m, k] w[n, k], on the gfx950 matrix cores in bfloat16
// with fp32 accumulation.
//
// Tiling: a 256-thread workgroup owns a 128 x 128 tile of y; each of its four waves owns a
// 64 x 64 quarter as 2 x 2 blocks of the 32x32x16 bf16 MFMA.  K is walked in steps of 64:
// the next x and w panels are fetched into registers while the current ones, double-buffered
// in LDS, feed the MFMAs, so one barrier per step suffices.  LDS rows are padded to 72 bf16
// (144 bytes, 36 banks apart), which keeps the 16-byte fragment reads of 16 consecutive rows
// on distinct banks.  fp32 x is rounded to bf16 (nearest, ties to even) on its way to LDS.
//
// Fragment layout of v_mfma_f32_32x32x16_bf16 (checked on the device): lane l supplies
// A[l % 32][8 (l / 32) .. +8] and B[8 (l / 32) .. +8][l % 32]; accumulator register r of lane
// l is C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].  With B = w^T the B fragment is eight
// consecutive k of w row (l % 32): both operands are row reads of their LDS panels.
//
// Tiles of one row block are consecutive in the workgroup order after the XCD remap below,
// so the six column tiles of a q/k/v projection read their x panel from one XCD's L2.
#include "linear.hpp"

#include "common.hpp"

namespace gat {
namespace {

typedef __bf16 lin_bf16x8 __attribute__((ext_vector_type(8)));
typedef float lin_f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kPitch = kBK + 8;               // bf16 elements per LDS row
constexpr int kLinThreads = 256;
constexpr int kXcds = 8;

__device__ __forceinline__ uint32_t to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;     // NaN stays a (quiet) NaN
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Workgroup b runs on XCD b % 8.  Give XCD x a contiguous range of tiles so that the column
// tiles of one row block run on one XCD, close in time.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t n_tiles) {
    const int64_t x = b % kXcds, j = b / kXcds;
    const int64_t q = n_tiles / kXcds, rem = n_tiles % kXcds;
    return x * q + (x < rem ? x : rem) + j;
}

// One 128 x 64 bf16 panel (rows r0.., k0..) of a [rows, K] bf16 matrix: 1024 16-byte pieces,
// four per thread; rows past `rows` and k past K read as zero.
struct PanelBf16 {
    uint4 v[4];
    __device__ __forceinline__ void fetch(const uint16_t* base, int64_t rows, int K, int64_t r0, int k0, int t) {
        const int c = (t & 7) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = r0 + (t >> 3) + 32 * i;
            v[i] = (r < rows && k0 + c < K) ? ld16(base + r * K + k0 + c) : make_uint4(0, 0, 0, 0);
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds, int t) const {
        const int c = (t & 7) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(lds + ((t >> 3) + 32 * i) * kPitch + c) = v[i];
    }
};

// The same panel read from an fp32 matrix: 2048 16-byte pieces, eight per thread, each
// rounded to four bf16 on the way to LDS.
struct PanelF32 {
    uint4 v[8];
    __device__ __forceinline__ void fetch(const float* base, int64_t rows, int K, int64_t r0, int k0, int t) {
        const int c = (t & 15) * 4;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t r = r0 + (t >> 4) + 16 * i;
            v[i] = (r < rows && k0 + c < K) ? ld16(base + r * K + k0 + c) : make_uint4(0, 0, 0, 0);
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds, int t) const {
        const int c = (t & 15) * 4;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint2 h;
            h.x = to_bf16_rne(__uint_as_float(v[i].x)) | (to_bf16_rne(__uint_as_float(v[i].y)) << 16);
            h.y = to_bf16_rne(__uint_as_float(v[i].z)) | (to_bf16_rne(__uint_as_float(v[i].w)) << 16);
            *reinterpret_cast<uint2*>(lds + ((t >> 4) + 16 * i) * kPitch + c) = h;
        }
    }
};

template <typename XPanel, typename XT, bool Y_BF16>
__global__ __launch_bounds__(kLinThreads, 2) void linear_kernel(const XT* __restrict__ x,
                                                                const uint16_t* __restrict__ w,
                                                                const float* __restrict__ bias, int64_t M, int K,
                                                                int N, LinearOut out, int64_t n_col_tiles,
                                                                int64_t n_tiles) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][kBM * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t ws[2][kBN * kPitch];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t tile = xcd_tile(blockIdx.x, n_tiles);
    const int64_t m0 = (tile / n_col_tiles) * kBM;
    const int n0 = static_cast<int>(tile % n_col_tiles) * kBN;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

    lin_f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    XPanel xp;
    PanelBf16 wp;
    xp.fetch(x, M, K, m0, 0, t);
    wp.fetch(w, N, K, n0, 0, t);
    xp.store(xs[0], t);
    wp.store(ws[0], t);
    __syncthreads();

    const int n_steps = (K + kBK - 1) / kBK;
    const int fr = lane & 31, fk = (lane >> 5) * 8;
    for (int s = 0; s < n_steps; ++s) {
        const int cur = s & 1;
        const bool more = s + 1 < n_steps;
        if (more) {
            xp.fetch(x, M, K, m0, (s + 1) * kBK, t);
            wp.fetch(w, N, K, n0, (s + 1) * kBK, t);
        }
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 16) {
            lin_bf16x8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const lin_bf16x8*>(&xs[cur][(wm + 32 * i + fr) * kPitch + kk + fk]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = *reinterpret_cast<const lin_bf16x8*>(&ws[cur][(wn + 32 * j + fr) * kPitch + kk + fk]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            xp.store(xs[cur ^ 1], t);
            wp.store(ws[cur ^ 1], t);
        }
        __syncthreads();
    }

    // epilogue: bias, split into the output arrays, fp32 or bf16 stores
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn + 32 * j + fr;
        if (col >= N) continue;
        const int seg = col / out.width, cc = col - seg * out.width;
        const float bv = bias ? bias[col] : 0.0f;
        char* base = static_cast<char*>(out.p[seg]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row >= M) continue;
                const float y = acc[i][j][r] + bv;
                const int64_t idx = row * out.width + cc;
                if (Y_BF16)
                    reinterpret_cast<uint16_t*>(base)[idx] = static_cast<uint16_t>(to_bf16_rne(y));
                else
                    reinterpret_cast<float*>(base)[idx] = y;
            }
        }
    }
}

template <typename XPanel, typename XT, bool Y_BF16>
hipError_t launch_typed(const void* x, const uint16_t* w, const float* bias, int64_t M, int K, int N,
                        const LinearOut& out, hipStream_t stream) {
    const int64_t n_col_tiles = (N + kBN - 1) / kBN;
    const int64_t n_tiles = (M + kBM - 1) / kBM * n_col_tiles;
    hipLaunchKernelGGL((linear_kernel<XPanel, XT, Y_BF16>), dim3(static_cast<uint32_t>(n_tiles)), dim3(kLinThreads),
                       0, stream, static_cast<const XT*>(x), w, bias, M, K, N, out, n_col_tiles, n_tiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_linear(const void* x, bool x_bf16, const uint16_t* w, const float* bias, int64_t M, int K, int N,
                         const LinearOut& out, bool y_bf16, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    if (x_bf16)
        return y_bf16 ? launch_typed<PanelBf16, uint16_t, true>(x, w, bias, M, K, N, out, stream)
                      : launch_typed<PanelBf16, uint16_t, false>(x, w, bias, M, K, N, out, stream);
    return y_bf16 ? launch_typed<PanelF32, float, true>(x, w, bias, M, K, N, out, stream)
                  : launch_typed<PanelF32, float, false>(x, w, bias, M, K, N, out, stream);
}

}  // namespace gat
