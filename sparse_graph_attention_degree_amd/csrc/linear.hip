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

typedef __bf16 lin_bf16x2 __attribute__((ext_vector_type(2)));
typedef float lin_f32x2 __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 bits (lo in the low half) with gfx950's v_cvt_pk_bf16_f32: round to
// nearest, ties to even; a NaN stays a NaN.
__device__ __forceinline__ uint32_t bf16_pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((lin_f32x2){lo, hi}, lin_bf16x2));
}

__device__ __forceinline__ uint32_t to_bf16_rne(float f) { return bf16_pack2(f, 0.0f) & 0xffffu; }

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
            const uint2 h = make_uint2(bf16_pack2(__uint_as_float(v[i].x), __uint_as_float(v[i].y)),
                                       bf16_pack2(__uint_as_float(v[i].z), __uint_as_float(v[i].w)));
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

// ------------------------------------------------------------------ stationary weights, K <= 256
// For in_dim <= 256 a wave keeps its w fragments for the whole of K in registers (2 column
// tiles x 16 k-steps = 128 AGPRs), so w is read once per workgroup and only x streams.  A
// 256-thread workgroup owns 256 output columns (one column group of 64 per wave, each wave
// covering the 32 rows of a block as one MFMA row tile) and walks a strided stream of 32-row
// blocks of x: blocks i + 1 and i + 2 wait in registers while block i, in LDS, feeds the MFMAs
// (each 16-byte fragment of x read from LDS feeds two MFMAs); then block i + 1 goes to the other
// LDS buffer and block i + 3 is fetched into its registers.  With bf16 x two workgroups share a
// CU (244 registers per lane, 51 KB of LDS each), so that one's epilogue and barriers overlap the
// other's MFMAs; 64-row blocks at one workgroup per CU ran the two phases back to back.
// Vector-memory waits count in issue order, so each fetch precedes the block's stores and the
// number of loads and stores per block is fixed (buffer accesses, no branches): waiting for a
// fetched block then leaves every later access in flight.  The results leave through a row-major
// LDS stage as whole 16-byte pieces of rows, with non-temporal stores.  The grid holds one or two
// workgroups per CU; the column blocks of one row stream are consecutive after the XCD remap, so
// the q, k and v workgroups of the same rows share one XCD's L2 copy of x.
constexpr int kWsK = 256;                  // largest in_dim of this path
constexpr int kWsKK = kWsK / 16;           // MFMA k-steps
// rows per block: one 32-row MFMA tile, for bf16 and fp32 x
template <bool XF32>
constexpr int ws_rows() { return 32; }
// Resident workgroups per CU: two where the registers allow (bf16 x, buffer stores: 244 of the
// 256 registers a lane may hold at two waves per SIMD), so that one workgroup's epilogue and
// barriers overlap the other's MFMAs; one otherwise.
template <bool XF32, bool BUF>
constexpr int ws_per_cu() { return !XF32 && BUF ? 2 : 1; }
constexpr int kWsCols = 256;               // columns per workgroup
constexpr int kWsThreads = 256;            // 4 column groups of 64
constexpr int kWsPitch = kWsK + 8;         // bf16 per LDS row (528 bytes: rows 4 banks apart)

typedef unsigned int lin_u32x4 __attribute__((ext_vector_type(4)));

// Blocks of x and y are addressed through buffer descriptors (base, size in bytes) rebuilt per
// block: a byte offset at or past the size reads 0 and drops a write, so edge rows and columns
// need no branches.
constexpr uint32_t kOob = 0x80000000u;
constexpr int kStoreNt = 2;                // cache-policy bit of a non-temporal store (gfx950)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t lin_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ uint4 lin_load16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    const lin_u32x4 v = __builtin_bit_cast(lin_u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool XF32>
struct RowBlock;

// 32 rows x 256 bf16 = 1024 pieces of 16 bytes, four per thread (32 threads per row)
template <>
struct RowBlock<false> {
    uint4 v[4];
    __device__ __forceinline__ void fetch(const void* xv, int64_t M, int K, int64_t r0, int t) {
        const int64_t rows = r0 >= M ? 0 : M - r0 < 32 ? M - r0 : 32;
        const auto rs = lin_rsrc(static_cast<const uint16_t*>(xv) + (rows > 0 ? r0 * K : 0),
                                 static_cast<uint32_t>(rows * K * 2));
        const int c = (t & 31) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t off = c < K ? static_cast<uint32_t>((((t >> 5) + 8 * i) * K + c) * 2) : kOob;
            v[i] = lin_load16(rs, off);
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds, int t) const {
        const int c = (t & 31) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(lds + ((t >> 5) + 8 * i) * kWsPitch + c) = v[i];
    }
};

// 32 rows x 256 fp32 = 2048 pieces, eight per thread (64 threads per row), rounded to bf16
template <>
struct RowBlock<true> {
    uint4 v[8];
    __device__ __forceinline__ void fetch(const void* xv, int64_t M, int K, int64_t r0, int t) {
        const int64_t rows = r0 >= M ? 0 : M - r0 < 32 ? M - r0 : 32;
        const auto rs = lin_rsrc(static_cast<const float*>(xv) + (rows > 0 ? r0 * K : 0),
                                 static_cast<uint32_t>(rows * K * 4));
        const int c = (t & 63) * 4;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t off = c < K ? static_cast<uint32_t>((((t >> 6) + 4 * i) * K + c) * 4) : kOob;
            v[i] = lin_load16(rs, off);
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds, int t) const {
        const int c = (t & 63) * 4;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint2 h = make_uint2(bf16_pack2(__uint_as_float(v[i].x), __uint_as_float(v[i].y)),
                                       bf16_pack2(__uint_as_float(v[i].z), __uint_as_float(v[i].w)));
            *reinterpret_cast<uint2*>(lds + ((t >> 6) + 4 * i) * kWsPitch + c) = h;
        }
    }
};

template <bool XF32, bool Y_BF16, bool BUF>
__global__ __launch_bounds__(kWsThreads, (ws_per_cu<XF32, BUF>())) void linear_wstat_kernel(const void* __restrict__ x,
                                                                     const uint16_t* __restrict__ w,
                                                                     const float* __restrict__ bias, int64_t M,
                                                                     int K, int N, LinearOut out, int n_col_blocks,
                                                                     int64_t n_streams, int64_t n_row_blocks,
                                                                     int vec) {
    static_assert(kWsThreads == kWsCols, "one bias entry per thread");
    constexpr int kRows = ws_rows<XF32>();
    constexpr int kTi = kRows / 32;                               // MFMA row tiles per block
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][kRows * kWsPitch];
    __shared__ __attribute__((aligned(16))) float bs[kWsCols];
    constexpr int kYB = Y_BF16 ? 2 : 4;                          // bytes per output element
    constexpr int kOsPitch = (kWsCols + 16 / kYB) * kYB;         // stage row bytes, padded by 16
    __shared__ __attribute__((aligned(16))) char ostage[kRows * kOsPitch];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t g = xcd_tile(blockIdx.x, gridDim.x);
    const int cb = static_cast<int>(g % n_col_blocks);
    const int64_t first = g / n_col_blocks;
    const int fr = lane & 31, fk = (lane >> 5) * 8;

    // The MFMA's A operand is w (32 output columns x 16 k) and its B operand x^T (16 k x 32 rows),
    // so the accumulator holds a tile of y^T: register 4 q + e of lane l is y[row l % 32]
    // [column 8 q + 4 (l / 32) + e], four consecutive columns of one row per lane, stored as one
    // vector.  This wave's two column tiles of w over the whole of K, zero past N and K:
    // All 16 k-steps run for any K <= 256: w fragments and the x block in LDS are zero past K,
    // so the steps past K add exact zeros.
    constexpr int NKK = kWsKK;
    lin_bf16x8 wf[2][NKK];
    {
        uint4 wv[2][NKK];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int wcol = cb * kWsCols + wave * 64 + 32 * j + fr;
            const bool cin = wcol < N;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const int k = kk * 16 + fk;
                wv[j][kk] = (cin && k < K) ? ld16(w + static_cast<int64_t>(wcol) * K + k) : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                lin_u32x4 u = {wv[j][kk].x, wv[j][kk].y, wv[j][kk].z, wv[j][kk].w};
                asm volatile("" : "+a"(u));           // keep w in AGPRs (an MFMA operand may live there)
                wf[j][kk] = __builtin_bit_cast(lin_bf16x8, u);
            }
    }
    {
        const int c = cb * kWsCols + t;
        bs[t] = (bias != nullptr && c < N) ? bias[c] : 0.0f;
    }

    int64_t blk = first;
    if (blk >= n_row_blocks) return;                  // uniform over the workgroup
    // Blocks p + 1 and p + 2 of this stream wait in registers (rb0, rb1 in turn) while block p is
    // computed from LDS: 64 KB of x in flight per CU.  A fetch past the last block reads nothing
    // (empty descriptor), so every step issues the same loads and stores.
    RowBlock<XF32> rb0, rb1;
    rb0.fetch(x, M, K, blk * kRows, t);
    rb0.store(xs[0], t);
    rb0.fetch(x, M, K, (blk + n_streams) * kRows, t);
    const auto none = lin_rsrc(out.p[0], 0);
    constexpr int kStores = kRows * (kWsCols * kYB / 16) / kWsThreads;     // epilogue stores per step
    // As many dropped stores (past an empty descriptor) as a step issues, so that every fetch is
    // followed by the same memory instructions on every path and its wait leaves them in flight.
    auto dummy_stores = [&]() {
        if (BUF) {
#pragma unroll
            for (int u = 0; u < kStores; ++u)
                __builtin_amdgcn_raw_buffer_store_b128((gat_v4i){0, 0, 0, 0}, none, kOob + 16 * u, 0, 0);
        }
    };
    dummy_stores();
    rb1.fetch(x, M, K, (blk + 2 * n_streams) * kRows, t);
    dummy_stores();
    __syncthreads();

    const int cl0 = wave * 64 + 4 * (lane >> 5);     // block-local column of this lane's first quad
    const int width = out.width;
    // one block: compute from xcur, move the next block from rbc to xnext, refill rbc three
    // blocks ahead, store the results; false after the stream's last block
    auto step = [&](RowBlock<XF32>& rbc, const uint16_t* xcur, uint16_t* xnext) -> bool {
        lin_f32x16 acc[kTi][2];                      // start from the bias: y = b + sum_k x w
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // accumulator register 4 q + e of tile j holds column cl0 + 32 j + 8 q + e
                const float4 b4 = *reinterpret_cast<const float4*>(&bs[cl0 + 32 * j + 8 * q]);
#pragma unroll
                for (int i = 0; i < kTi; ++i) {
                    acc[i][j][4 * q] = b4.x;
                    acc[i][j][4 * q + 1] = b4.y;
                    acc[i][j][4 * q + 2] = b4.z;
                    acc[i][j][4 * q + 3] = b4.w;
                }
            }
        const uint16_t* arow = &xcur[fr * kWsPitch + fk];
        lin_bf16x8 a[2][kTi];                        // fragments of step kk (kk & 1) and kk + 1
#pragma unroll
        for (int i = 0; i < kTi; ++i) a[0][i] = *reinterpret_cast<const lin_bf16x8*>(arow + 32 * i * kWsPitch);
        // raised issue priority while the MFMAs go out: the other workgroup's epilogue on this
        // SIMD fills the gaps instead of delaying them
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const int c = kk & 1;
            if (kk + 1 < NKK) {
#pragma unroll
                for (int i = 0; i < kTi; ++i)
                    a[c ^ 1][i] = *reinterpret_cast<const lin_bf16x8*>(arow + 32 * i * kWsPitch + (kk + 1) * 16);
            }
#pragma unroll
            for (int i = 0; i < kTi; ++i) {
                acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[0][kk], a[c][i], acc[i][0], 0, 0, 0);
                acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[1][kk], a[c][i], acc[i][1], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        const int64_t nxt = blk + n_streams;
        const bool more = nxt < n_row_blocks;
        if (more) rbc.store(xnext, t);
        rbc.fetch(x, M, K, (nxt + 2 * n_streams) * kRows, t);
        // Epilogue through LDS: the accumulators (plus bias, rounded if bf16) go to a row-major
        // stage, then every thread stores whole 16-byte pieces of consecutive columns, so one wave
        // instruction writes 1 KB of complete rows.
#pragma unroll
        for (int i = 0; i < kTi; ++i) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int cl = cl0 + 32 * j + 8 * q;
                    const float y0 = acc[i][j][4 * q], y1 = acc[i][j][4 * q + 1];
                    const float y2 = acc[i][j][4 * q + 2], y3 = acc[i][j][4 * q + 3];
                    char* dst = ostage + (32 * i + fr) * kOsPitch + cl * kYB;
                    if (Y_BF16)
                        *reinterpret_cast<uint2*>(dst) = make_uint2(bf16_pack2(y0, y1), bf16_pack2(y2, y3));
                    else
                        *reinterpret_cast<float4*>(dst) = make_float4(y0, y1, y2, y3);
                }
            }
        }
        __syncthreads();
        {
            constexpr int kEpp = 16 / kYB;                       // columns per 16-byte piece
            constexpr int kPiecesPerRow = kWsCols / kEpp;
            constexpr int kRowsPerPass = kWsThreads / kPiecesPerRow;
            const int cl = (t % kPiecesPerRow) * kEpp;
            const int c = cb * kWsCols + cl;
            if (BUF) {
                // every column of this workgroup lies in one output array
                const int cbase = cb * kWsCols;
                const int seg = (cbase >= width) + (cbase >= 2 * width);
                char* p = static_cast<char*>(seg == 0 ? out.p[0] : (seg == 1 ? out.p[1] : out.p[2]));
                const int64_t r0 = blk * kRows;
                const int64_t rows = M - r0 < kRows ? M - r0 : kRows;
                const auto rs = lin_rsrc(p + r0 * width * kYB, static_cast<uint32_t>(rows * width * kYB));
                const int cc = c - seg * width;
#pragma unroll
                for (int u = 0; u < kRows / kRowsPerPass; ++u) {
                    const int rl = t / kPiecesPerRow + kRowsPerPass * u;
                    const uint32_t off = c + kEpp <= N ? static_cast<uint32_t>((rl * width + cc) * kYB) : kOob;
                    const uint4 v = *reinterpret_cast<const uint4*>(ostage + rl * kOsPitch + cl * kYB);
                    // non-temporal: the outputs are not read again by this kernel
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(gat_v4i, (lin_u32x4){v.x, v.y, v.z, v.w}),
                                                           rs, off, 0, kStoreNt);
                }
            } else {
#pragma unroll
                for (int u = 0; u < kRows / kRowsPerPass; ++u) {
                    const int rl = t / kPiecesPerRow + kRowsPerPass * u;
                    const int64_t row = blk * kRows + rl;
                    if (row >= M || c >= N) continue;
                    const char* src = ostage + rl * kOsPitch + cl * kYB;
                    if (vec && c + kEpp <= N) {
                        const int seg = (c >= width) + (c >= 2 * width);
                        char* p = static_cast<char*>(seg == 0 ? out.p[0] : (seg == 1 ? out.p[1] : out.p[2]));
                        *reinterpret_cast<uint4*>(p + (row * width + (c - seg * width)) * kYB) =
                            *reinterpret_cast<const uint4*>(src);
                    } else {
                        for (int e = 0; e < kEpp && c + e < N; ++e) {
                            const int ce = c + e;
                            const int seg = (ce >= width) + (ce >= 2 * width);
                            char* p = static_cast<char*>(seg == 0 ? out.p[0] : (seg == 1 ? out.p[1] : out.p[2]));
                            char* d = p + (row * width + (ce - seg * width)) * kYB;
                            if (Y_BF16)
                                *reinterpret_cast<uint16_t*>(d) = *reinterpret_cast<const uint16_t*>(src + e * kYB);
                            else
                                *reinterpret_cast<float*>(d) = *reinterpret_cast<const float*>(src + e * kYB);
                        }
                    }
                }
            }
        }
        if (!more) return false;
        __syncthreads();
        blk = nxt;
        return true;
    };
    for (;;) {
        if (!step(rb0, xs[0], xs[1])) break;
        if (!step(rb1, xs[1], xs[0])) break;
    }
}

template <bool XF32, bool Y_BF16>
hipError_t launch_wstat(const void* x, const uint16_t* w, const float* bias, int64_t M, int K, int N,
                        const LinearOut& out, hipStream_t stream) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int n_col_blocks = (N + kWsCols - 1) / kWsCols;
    const int64_t n_row_blocks = (M + ws_rows<XF32>() - 1) / ws_rows<XF32>();
    // 16-byte stores need pieces that do not straddle output arrays, and aligned arrays (1); the
    // buffer stores also need each workgroup's 256 columns inside one array (2)
    const int n_out = N / out.width;
    bool aligned = true;
    for (int s = 0; s < n_out; ++s) aligned = aligned && reinterpret_cast<uintptr_t>(out.p[s]) % 16 == 0;
    const int vec = !aligned ? 0 : out.width % kWsCols == 0 ? 2 : out.width % (Y_BF16 ? 8 : 4) == 0 ? 1 : 0;
    const int per_cu = vec == 2 ? ws_per_cu<XF32, true>() : ws_per_cu<XF32, false>();
    int64_t n_streams = (int64_t)per_cu * cus / n_col_blocks;
    if (n_streams < 1) n_streams = 1;
    if (n_streams > n_row_blocks) n_streams = n_row_blocks;
    const int64_t grid = n_streams * n_col_blocks;
    if (vec == 2)
        hipLaunchKernelGGL((linear_wstat_kernel<XF32, Y_BF16, true>), dim3(static_cast<uint32_t>(grid)),
                           dim3(kWsThreads), 0, stream, x, w, bias, M, K, N, out, n_col_blocks, n_streams,
                           n_row_blocks, vec);
    else
        hipLaunchKernelGGL((linear_wstat_kernel<XF32, Y_BF16, false>), dim3(static_cast<uint32_t>(grid)),
                           dim3(kWsThreads), 0, stream, x, w, bias, M, K, N, out, n_col_blocks, n_streams,
                           n_row_blocks, vec);
    return hipGetLastError();
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
    if (K <= kWsK) {
        if (x_bf16)
            return y_bf16 ? launch_wstat<false, true>(x, w, bias, M, K, N, out, stream)
                          : launch_wstat<false, false>(x, w, bias, M, K, N, out, stream);
        return y_bf16 ? launch_wstat<true, true>(x, w, bias, M, K, N, out, stream)
                      : launch_wstat<true, false>(x, w, bias, M, K, N, out, stream);
    }
    if (x_bf16)
        return y_bf16 ? launch_typed<PanelBf16, uint16_t, true>(x, w, bias, M, K, N, out, stream)
                      : launch_typed<PanelBf16, uint16_t, false>(x, w, bias, M, K, N, out, stream);
    return y_bf16 ? launch_typed<PanelF32, float, true>(x, w, bias, M, K, N, out, stream)
                  : launch_typed<PanelF32, float, false>(x, w, bias, M, K, N, out, stream);
}

}  // namespace gat
