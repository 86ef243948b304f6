// Node projections on the matrix cores: y = x . w^T + bias (nn.Linear, weights [out, in]).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gat {

constexpr int kLinMaxOut = 3;          // output arrays one call can split y into

struct LinearOut {
    void* p[kLinMaxOut];               // out[s] holds y's columns [s * width, (s + 1) * width)
    int width;                         // columns per output array
};

// x [M,K] fp32 (x_bf16 = false; rounded to bf16 on load) or bf16 bits; w [N,K] bf16 bits;
// bias [N] fp32 or null; y written as fp32 or bf16 (y_bf16).  Requires K % 8 == 0, 16-byte
// aligned x and w, N = n_out * out.width.
hipError_t launch_linear(const void* x, bool x_bf16, const uint16_t* w, const float* bias, int64_t M, int K, int N,
                         const LinearOut& out, bool y_bf16, hipStream_t stream);

}  // namespace gat
