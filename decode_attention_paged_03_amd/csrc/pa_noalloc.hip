// pa_noalloc.hip -- the device scratch array behind pa_decode_noalloc().
//
// Some callers cannot allocate device memory around a decode step: code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc.  For them the library keeps
// its own workspace, one file-scope device array of kNoallocScratchBytes that every GPU the
// library runs on holds until the process ends.  On the host, the array's name denotes a
// host-side stand-in, not device memory, so it is never passed to a kernel or a copy: the
// first call on a device, with that device current, asks the runtime for the array's device
// address and keeps it per device (each GPU holds its own copy at its own address).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "pa_internal.h"

namespace pa {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];   // device address per device; null: not looked up
}  // namespace

bool noalloc_scratch(void** ptr, size_t* bytes) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return false;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return false;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    *bytes = kNoallocScratchBytes;
    return true;
}

}  // namespace pa
