// scratch.hip - the library's one static device buffer: the routing workspace
// of moe_dispatch_noalloc, for callers that cannot allocate device memory.
//
// Each GPU the library runs on holds one copy (kScratchBytes) from the first
// noalloc call on it until the process ends.  Host code never uses the array's
// name as an address: on the host it only names the symbol.  The device
// address of each GPU's copy is looked up once, with that GPU current, and kept
// per device; every later use (the kernels' workspace argument) goes through
// that address.  Every noalloc call on a GPU shares its copy, so two such calls
// that can overlap on one GPU (different streams) race.  Nothing in it needs
// clearing: the routing's arrival ticket carries a tag and repairs a word
// without it (the array starts as zeros), and every other word is written
// before it is read within a call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.hpp"

namespace moe {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of scratch on each GPU, once looked up

}  // namespace

hipError_t scratch_for_stream(hipStream_t s, void** out) {
    hipDevice_t dev = 0;
    hipError_t e = hipStreamGetDevice(s, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return e;
        if (back != hipSuccess) return back;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace moe
