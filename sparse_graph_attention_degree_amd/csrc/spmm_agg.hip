// Instantiation of the aggregation engine (spmm.hpp) for mode kAgg; one
// translation unit per mode so the three compile in parallel.
#include "spmm.hpp"

namespace gat {

hipError_t launch_spmm_agg(int dtype, int H, int D, const int32_t* row_ptr, const int32_t* col, int64_t n_rows,
                          int64_t n_src, const float* sc, const void* q, const void* k, const void* v, float scale, float* out,
                          const PlanView* plan, hipStream_t stream) {
    return launch_spmm_mode<kAgg>(dtype, H, D, row_ptr, col, n_rows, n_src, sc, q, k, v, scale, out, plan, stream);
}

}  // namespace gat
