// Streaming a contiguous run of floats through one wave with raw buffer accesses.
//
// A buffer descriptor over [p, p + bytes) lives in scalar registers (so the run must be the same
// for every lane of the wave: build it from wave-uniform values, or the compiler wraps each access
// in a readfirstlane loop).  A load past the end reads 0 without touching memory and a store past
// it is dropped, so a partial tail needs no per-lane branch; each access costs one 32-bit lane
// offset (plus an immediate) instead of a 64-bit address.
#pragma once

#include "common.hpp"

namespace gat {

// bytes < 2^31 (the descriptor's record count is 32-bit; every caller passes one run or chunk of at
// most a few KB)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span(const float* p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, (int)bytes, 0x00020000);
}
// off: byte offset of this lane's element.  It is passed as the lane offset (with a constant
// part the compiler folds into the instruction's immediate offset), both of which the range
// check covers; the scalar offset stays 0.
__device__ __forceinline__ float bload(__amdgpu_buffer_rsrc_t r, int off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, float v, int off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}

// x, with its value hidden from the optimiser at this point.  Inside a loop, the lane offsets of
// an unrolled run are then computed from it in the loop body, where instruction selection folds
// each constant part into the access's immediate offset.  Without it, loop-invariant code motion
// hoists every (offset + constant) out of the loop, one VGPR each (16 of them for a 16-element
// run), and the kernel's occupancy drops.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// The same for a wave-uniform 32-bit count (a chunk length computed from 64-bit sizes): without it
// the compiler may keep the count 64-bit and compare it with each unrolled k * 64 as a 64-bit
// constant, held in a VGPR pair.
__device__ __forceinline__ int opaque_uniform(int x) {
    asm volatile("" : "+s"(x));
    return x;
}

}  // namespace gat
