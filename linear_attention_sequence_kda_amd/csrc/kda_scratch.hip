// kda_scratch.hip -- the static device buffer behind kda_chunk_fwd_noalloc.
//
// The allocation-free prefill keeps its work memory (the records of one span
// of chunks and, with several spans and no S_final, the state between spans)
// in this file-scope array instead of a caller workspace.  Every GPU the
// library runs on holds its own copy, at its own address, until the process
// ends; calls on one GPU share it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda.h"
#include "kda_internal.h"

namespace kda {

static __device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

// In host code `scratch` names a host-side stand-in, not device memory: the
// device address is looked up once per device, with that device current, and
// kept; kernels and copies only ever see that address.
hipError_t scratch_address(void** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* ptrs[kMaxDevices] = {};
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        ptrs[dev] = p;
    }
    *out = ptrs[dev];
    return hipSuccess;
}

}  // namespace kda
