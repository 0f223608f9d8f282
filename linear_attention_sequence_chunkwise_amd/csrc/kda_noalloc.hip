// kda_noalloc.hip -- the static device scratch array behind kda_prefill_fwd_noalloc.
//
// Callers that cannot allocate device memory get the prefill's workspace (the varlen chunk
// table and the factor blocks) from this fixed array instead of a buffer of their own.  Each
// device holds its own copy from the library's load until the process ends.  In host code the
// name `scratch` is only a host-side stand-in for the symbol: the kernels are given the device
// address that hipGetSymbolAddress returns for the current device, never the name itself.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda.h"
#include "kda_launch.h"

static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace kda {

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_addr[kMaxDevices];
hipError_t g_status[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    // once per device, with that device current (it is: hipGetDevice just returned it)
    std::call_once(g_once[dev], [dev] {
        void* p = nullptr;
        g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_addr[dev] = g_status[dev] == hipSuccess ? p : nullptr;
    });
    if (g_status[dev] != hipSuccess) return g_status[dev];
    *ptr = g_addr[dev];
    return hipSuccess;
}

}  // namespace kda
