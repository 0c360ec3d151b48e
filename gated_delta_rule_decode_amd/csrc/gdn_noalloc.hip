// gdn_noalloc.hip -- the static device array behind gdn_prefill_chunked_noalloc.
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) get the prefill with
// its workspace in this file-scope array instead of a caller buffer.  Every
// GPU the library runs on holds its own copy of the array until the process
// ends.  In host code the array's name is only a stand-in for the symbol, so
// its device address is looked up once per device, with that device current,
// and kept; kernels receive that address, never the name.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

static __device__ __attribute__((aligned(256))) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device ordinal

}  // namespace

namespace gdn {

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
    *ptr = nullptr;
    *bytes = 0;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    *bytes = GDN_NOALLOC_SCRATCH_BYTES;
    return hipSuccess;
}

}  // namespace gdn
