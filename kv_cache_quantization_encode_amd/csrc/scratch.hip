// Library-owned attention workspace for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc): a file-scope device array, one copy per GPU, held until
// the process ends.  Its address on each device comes from hipGetSymbolAddress
// (the array's name in host code is only a host-side stand-in), taken once per
// device while that device is current and kept per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace tq {

// Zero when the code object loads.  Every attention call leaves the barrier
// counters of the single-launch path back at zero, and the two-pass path needs
// no initial contents, so consecutive calls need no clearing.  Calls that
// overlap on one GPU share this memory and race.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

int scratch_prepare(int device) {
    if (device < 0 || device >= kMaxScratchDevices) return int(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[device]) return int(hipSuccess);
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return int(e);
    if (cur != device) return int(hipErrorInvalidDevice);
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return int(e != hipSuccess ? e : hipErrorInvalidSymbol);
    g_scratch_ptr[device] = p;
    return int(hipSuccess);
}

void *scratch_device_ptr(int device) {
    if (device < 0 || device >= kMaxScratchDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    return g_scratch_ptr[device];
}

}  // namespace tq
