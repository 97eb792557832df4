// mx_static.hip -- the one fixed device buffer of libmx, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc): mx_moe_linear_noalloc uses it as the
// workspace of the grouped GEMV's top-k combine.
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  In host code
// the array's name is only a host-side stand-in, so host code never passes
// it to a kernel or a copy: static_scratch() looks up the device address of
// the current device's copy once per device (with that device current) and
// every user takes that pointer.  Calls that use it on one GPU share it, and
// calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "mx_kernels.h"

namespace {

static __device__ __align__(256) unsigned char scratch[mx::kStaticScratchBytes];

// per device ordinal: the device address of its copy of scratch (0: not yet
// looked up; the zero-initialized state is valid before any constructor runs)
std::atomic<uintptr_t> g_scratch_ptr[64];

}  // namespace

namespace mx {

void *static_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    const uintptr_t known = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (known) return reinterpret_cast<void *>(known);
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev].store(reinterpret_cast<uintptr_t>(ptr), std::memory_order_release);
    return ptr;
}

}  // namespace mx
