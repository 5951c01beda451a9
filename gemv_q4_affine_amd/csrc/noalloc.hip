// noalloc.hip -- a fixed device scratch array for q4_gemm_image_noalloc, the
// entry point for callers that cannot allocate device memory.
//
// The array holds what q4_gemm_image keeps in its workspace: the binary16 X
// image and, for launches with few tiles, the split-K partial results.  Each
// GPU the library runs on holds its own copy from module load until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host that name is only a stand-in): the device address of this GPU's copy is
// looked up once per device, with that device current, and used from then on.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kernels.hpp"
#include "q4.h"

namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[Q4_NOALLOC_SCRATCH_BYTES];

std::mutex g_lookup_mu;
std::atomic<void*> g_scratch_addr[kMaxDevices];

}  // namespace

namespace q4 {

hipError_t noalloc_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lk(g_lookup_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (p == nullptr) return hipErrorInvalidSymbol;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace q4
