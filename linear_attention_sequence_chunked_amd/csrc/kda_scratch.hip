// kda_scratch.hip -- the library's one fixed device buffer, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops, harnesses that
// forbid allocation).  It backs the workspace of kda_chunk_prefill_segmented_noalloc.
//
// The array is a file-scope device variable: every GPU the library runs on holds its own
// copy, at its own address, from the time the code object is loaded until the process
// ends.  In host code the name `scratch` is only a host-side stand-in, never a device
// address; scratch_address() resolves the device address once per device (with that
// device current) and every later use goes through the resolved pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_launch.h"

namespace kda {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(void** out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace kda
