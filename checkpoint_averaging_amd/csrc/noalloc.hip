// Library-owned scratch for the allocation-free outer orthogonal step
// (dl_outer_orthogonal_step_noalloc), for callers that cannot allocate
// device memory: code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc.
//
// The scratch is one file-scope device array.  Every GPU the library runs the
// entry point on holds its own copy until the process ends.  This file holds
// nothing else, and the runtime loads a code object on first use, so a
// process that never calls the entry point does not hold the array (on
// MI355X the free device memory drops by 196 MiB at the first call, not
// before).  In host code `scratch` names a host-side stand-in, not
// device memory: its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that address is
// ever handed to kernels or runtime calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "noalloc.h"

namespace {

static __device__ __align__(256) unsigned char scratch[dlk::kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

namespace dlk {

hipError_t noalloc_scratch(int device, void** addr) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_addr[device] == nullptr) {
        int current = -1;
        if (hipError_t e = hipGetDevice(&current)) return e;
        if (current != device) return hipErrorInvalidDevice;   // the device must be current
        void* p = nullptr;
        if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return e;
        g_addr[device] = p;
    }
    *addr = g_addr[device];
    return hipSuccess;
}

}  // namespace dlk
