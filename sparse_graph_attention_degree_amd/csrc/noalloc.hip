// Library-owned device scratch for the entry point that allocates nothing
// (gat_fused_layer_noalloc in gat.h).  The degree-binning plan of such a call -- counts,
// per-block binner counts, segment and hub tables, hub partial states -- lives in one file-scope
// device array instead of a caller workspace.  Every GPU the library runs on holds its own copy
// of the array (GAT_NOALLOC_SCRATCH_BYTES) from the first such call until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device address is
// looked up once per device with hipGetSymbolAddress (that device current) and kept per device;
// host code only ever passes that address on.
#include <mutex>

#include "gat.h"
#include "kernels.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[GAT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_addr[kMaxDevices];   // device address of `scratch` on each device (null until looked up)

}  // namespace

namespace gat {

hipError_t noalloc_scratch(void** addr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> hold(g_lock);
    if (g_addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_addr[dev] = p;
    }
    *addr = g_addr[dev];
    return hipSuccess;
}

}  // namespace gat
