// kda_noalloc.cpp - the scratch of kda_prefill_noalloc: a file-scope device
// array that stands in for the workspace a caller would otherwise allocate
// (the chunked MFMA path's per-chunk operand records and, for packed
// sequences, its chunk offsets; no other kernel of the library uses scratch).
//
// In host code `scratch` names a host-side stand-in, not the device array, so
// its device address is taken once per device with hipGetSymbolAddress, with
// that device current, and only that address is ever handed to kernels.  Each
// GPU that loads the library holds its own copy until the process ends, and
// every call on one GPU shares it: calls that overlap in time on one GPU race.
// No part of it has to start at zero: within a call the kernels write every
// byte of it they read.
#include <mutex>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` per device; null until taken

}  // namespace

hipError_t noalloc_scratch(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
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
