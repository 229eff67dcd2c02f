// The library's static scratch buffer, for the entry points that allocate
// nothing (txl_relattn_fwd_noalloc): the key-split partial outputs live in a
// file-scope device array instead of a caller workspace.  Every device the
// library runs on holds its own copy (kScratchBytes) until the process ends.
//
// In host code the array's name is only a host-side stand-in; its device
// address comes from hipGetSymbolAddress, taken once per device (with that
// device current) on the first call there and kept per device.

#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[txl::kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];   // device address of `scratch` on each device, once taken

}  // namespace

namespace txl {

hipError_t scratch_buffer(void **ptr, size_t *bytes)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    *bytes = kScratchBytes;
    return hipSuccess;
}

}  // namespace txl
