// sparse_mla without a caller workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The split partials that dsa_sparse_mla keeps in the
// caller's workspace live here in a fixed device array instead; the kernels
// are sparse_mla's own, given that array's address.
//
// The array's address on a device is resolved with hipGetSymbolAddress the
// first time the entry point runs on that device (with the device current)
// and kept per device; host code never uses the array's name as an address.
// Every call on a device shares that device's copy: calls that overlap on one
// GPU race.  Nothing in it needs to start at zero (an empty split's partial
// is never read, only its (m, l) pair, which every split writes).
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "dsa_common.h"
#include "dsa_launch.h"

namespace dsa {

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

}  // namespace dsa

namespace dsa_host {

namespace {
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // per device: the address of dsa::scratch, null until resolved
}  // namespace

hipError_t noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(dsa::scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace dsa_host
