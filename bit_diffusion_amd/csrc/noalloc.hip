// noalloc.hip -- the device-resident scratch of svdq_gemm_w4a4_packed_noalloc, the packed
// GEMM for callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The K split's partial tiles go to `scratch`, a file-scope device array of
// kSplitWorkspaceMax bytes (the most the split ever uses), which every GPU the library
// runs on holds until the process ends.  In host code the array's name is only a host-side
// stand-in, so its device address is looked up once per device with hipGetSymbolAddress
// (that device current) and kept; kernels only ever receive that address.  Every call on a
// GPU shares its array: calls that overlap on one GPU (different streams, no ordering
// between them) race on it.  Nothing in it must start at zero: each split stores its whole
// partial tile before the fixed-order sum reads it, in stream order.
#include <mutex>

#include <hip/hip_runtime.h>

#include "launch.hpp"

namespace {

__device__ __align__(256) float scratch[svdq::kSplitWorkspaceMax / 4];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace svdq {

hipError_t noalloc_scratch(void** ptr, int64_t* bytes) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    *bytes = (int64_t)sizeof(scratch);
    return hipSuccess;
}

}  // namespace svdq
