// Device-side building blocks shared by the gfx950 kernels of libgat.
//
// Lane geometry.  A feature row of one node is H*D elements (H heads x D dims),
// RB = H*D*sizeof(T) bytes.  It is read in 16-byte pieces (global_load_dwordx4):
// NPC = RB/16 pieces.  A "slot" is the group of G = min(64, NPC) lanes that holds
// one row; a wave64 holds P = 64/G slots, and each lane of a slot holds
// NV = NPC/G pieces (piece index v*G + q for lane q of the slot).  A piece never
// straddles two heads because D*sizeof(T) >= 32 bytes.
//
// Score layout.  A slot also reads edge scores [E,H] (edge-major) G values at a
// time: lane q holds edge (chunk start + q/H), head q%H, so a chunk covers
// SC = G/H edges and one coalesced dword load per lane fetches it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gat {

constexpr int kWave = 64;
constexpr int kBlock = 256;            // threads per workgroup in every kernel
constexpr int kWavesPerBlock = kBlock / kWave;

using bf16_t = uint16_t;                // raw bfloat16 bits

template <typename T>
struct Elem;
template <>
struct Elem<float> { static constexpr int bytes = 4; };
template <>
struct Elem<bf16_t> { static constexpr int bytes = 2; };

// GMAX caps the slot width: narrower slots put more rows in flight per wave, each lane then
// holding more pieces of its row.
template <typename T, int H_, int D_, int GMAX = kWave>
struct Geo {
    static constexpr int H = H_;
    static constexpr int D = D_;
    static constexpr int HD = H * D;
    static constexpr int S = Elem<T>::bytes;
    static constexpr int RB = HD * S;               // bytes per feature row
    static constexpr int NPC = RB / 16;             // 16-byte pieces per row
    static constexpr int GW = GMAX < kWave ? GMAX : kWave;
    static constexpr int G0 = NPC < GW ? NPC : GW;
    static constexpr int G = G0 < H ? H : G0;       // lanes per slot (at least one per head)
    static constexpr int P = kWave / G;             // slots per wave
    static constexpr int NV = NPC / G;              // pieces per lane
    static constexpr int EPP = 16 / S;              // elements per piece
    static constexpr int LPH = D * S / 16;          // pieces per head
    static constexpr int SC = G / H;                // edges per score chunk
    static_assert(D * S >= 32, "a head must span at least two pieces");
    static_assert(G % H == 0 && SC >= 1, "score chunk must hold whole edges");
    static_assert(NPC % G == 0, "pieces must tile the lanes");
};

// ---------------------------------------------------------------------------- lane helpers
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float shfl(float v, int src) { return __shfl(v, src); }
__device__ __forceinline__ int shfl(int v, int src) { return __shfl(v, src); }
__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask); }
__device__ __forceinline__ int shfl_xor(int v, int mask) { return __shfl_xor(v, mask); }

// DPP move within the wave (row_mask = bank_mask = 0xF; every source lane below is valid).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over each aligned group of N consecutive lanes (N a power of two <= 64); every lane of
// the group receives the sum.  Up to 16 lanes it stays in registers (DPP): two quad
// permutations give the quad sum, the half-row mirror (lane i <-> 7-i) adds the other quad,
// the row mirror (lane i <-> 15-i) adds the other half-row; wider groups use shuffles.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (N >= 2) x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
    if constexpr (N >= 4) x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
    if constexpr (N >= 8) x += dpp<0x141>(x);   // row_half_mirror
    if constexpr (N >= 16) x += dpp<0x140>(x);  // row_mirror
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    if constexpr (N >= 64) x += __shfl_xor(x, 32);
    return x;
}

// Hand-off point between the lanes of one wave through LDS: a value one lane wrote is read by
// another lane after this point, or an area other lanes read before this point is rewritten
// after it.  A wave's LDS instructions execute in issue order, so the hardware needs no wait;
// the two wave-scope fences keep the compiler from moving memory accesses across the point
// (without them only its failure to prove two lanes' addresses distinct keeps the order).
__device__ __forceinline__ void wave_lds_handoff() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// e^x as the hardware exp2 of x*log2(e).  exp(-inf) = 0.
__device__ __forceinline__ float exp_fast(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// ---------------------------------------------------------------------------- memory
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ void st16(void* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// widen one 16-byte piece to EPP floats (bf16 -> fp32 is exact: the bits move up 16 places)
template <typename T>
__device__ __forceinline__ void unpack(const uint4& v, float* f);

template <>
__device__ __forceinline__ void unpack<float>(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
}

template <>
__device__ __forceinline__ void unpack<bf16_t>(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16);
    f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16);
    f[7] = __uint_as_float(v.w & 0xffff0000u);
}

// ---------------------------------------------------------------------------- gathered tables
// A feature table of rows of RB bytes, read 16 bytes at a time.
//  Tab32: the table spans < 4 GiB.  Rows are read with buffer loads: the descriptor (base,
//         size) sits in scalar registers and each lane supplies one 32-bit byte offset, so a
//         gather costs one address instruction; an offset past the end reads 0.  The
//         descriptor's fourth dword (0x00020000) is the gfx9-family raw-buffer format.
//  Tab64: any size; 64-bit addresses.
typedef int gat_v4i __attribute__((ext_vector_type(4)));

template <int RB>
struct Tab32 {
    __amdgpu_buffer_rsrc_t rs;
    __device__ __forceinline__ Tab32(const void* base, int64_t n_rows)
        : rs(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)(uint32_t)(n_rows * RB),
                                                0x00020000)) {}
    __device__ __forceinline__ uint4 row16(int r, uint32_t byte_off) const {
        const gat_v4i x = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)r * (uint32_t)RB + byte_off, 0, 0);
        return make_uint4((uint32_t)x.x, (uint32_t)x.y, (uint32_t)x.z, (uint32_t)x.w);
    }
};

template <int RB>
struct Tab64 {
    const char* base;
    __device__ __forceinline__ Tab64(const void* b, int64_t) : base(static_cast<const char*>(b)) {}
    __device__ __forceinline__ uint4 row16(int r, uint32_t byte_off) const {
        return ld16(base + (int64_t)r * RB + byte_off);
    }
};

// ---------------------------------------------------------------------------- plan view
// Device view of a degree-binning plan (see gat_plan in gat.h).
struct PlanView {
    const int32_t* counts;    // [0] n_segments [1] n_hub_segments [2] n_hubs [3] n_long [4] overflow
    const int4* segs;         // (row, e_begin, e_end, slot)
    const int4* hubs;         // (row, first segment, n segments, 0)
    float* partials;          // [hub segment][state_floats]
    int64_t state_floats;
    int64_t seg_capacity;     // bounds on the table sizes (grid caps of the persistent kernels)
    int64_t hub_capacity;
    int64_t hubseg_capacity;
    int32_t short_max;        // rows with deg <= short_max belong to the lane-group kernels
    int32_t seg_len;
};

// Grid cap of the persistent kernels: 256 CUs x 8 workgroups.
constexpr int64_t kPersistentBlocks = 2048;
// Grid cap of the kernels over the plan's segment table (sized by the table's capacity; workgroups
// past the real count exit at once): up to this many, about one segment (or one hub segment) per
// workgroup or wave.  Segments differ in length by up to seg_len / short_max, and the hardware
// dispatcher balances them across the CUs better than a fixed stride over a resident grid.
constexpr int64_t kSegmentGrid = 65536;
// Grid cap of the per-edge gather kernels (SDDMM, edge_dot): one step of edges per wave up to
// 2^29 edges at 16 edges per step, a grid-stride loop beyond (2^23 workgroups x 256 work-items
// keeps the dispatch's 32-bit work-item count in range).  At 2^26 edges a grid of 65536
// workgroups looping over the edges took 7.09 ms against 6.77 ms.
constexpr int64_t kEdgeGridDefault = int64_t(1) << 23;
// The cap in force: kEdgeGridDefault unless gat_testing_edge_grid_cap lowered it (tests use that to
// run the grid-stride loop at sizes they can check).  Host only.
int64_t edge_grid_cap();

// kOverflow: 1 when the row degrees sum past the capacities the host sized from n_edges (row_ptr
// breaks its precondition row_ptr[n_rows] = n_edges); the binner then leaves every table empty.
enum CountIdx { kNSegs = 0, kNHubSegs = 1, kNHubs = 2, kNLong = 3, kOverflow = 4 };

}  // namespace gat
