// Scratch memory for pa_decode_noalloc: the split-context partials live in a
// file-scope device array instead of a caller's workspace, for callers that
// cannot allocate (code under graph capture, tight serving loops).  Each GPU
// the library runs on holds its own copy of the array, at its own address,
// until the process ends.  Host code never uses the array's name as an
// address: it asks HIP for the current device's copy once per device and
// passes that pointer to the kernels like any workspace.
#include <hip/hip_runtime.h>

#include <atomic>
#include <string>

#include "hip_util.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kScratchDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

}  // namespace

pa_status noalloc_scratch(void **out, std::string *why) {
    static std::atomic<void *> cache[kScratchDevices];
    int dev = 0;
    pa_status st = hip_status(hipGetDevice(&dev), why, "decode_noalloc: hipGetDevice");
    if (st != PA_OK) return st;
    if (dev < 0 || dev >= kScratchDevices) {
        if (why) *why = "decode_noalloc: device index out of range";
        return PA_ERR_UNSUPPORTED;
    }
    void *p = cache[dev].load(std::memory_order_acquire);
    if (!p) {  // first call on this device, with it current
        st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), why,
                        "decode_noalloc: hipGetSymbolAddress");
        if (st != PA_OK) return st;
        if (!p) {
            if (why) *why = "decode_noalloc: no address for the scratch array";
            return PA_ERR_HIP;
        }
        cache[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return PA_OK;
}

}  // namespace pa
