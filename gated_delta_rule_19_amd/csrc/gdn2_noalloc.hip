// Workspace for gdn2_chunk_fwd_noalloc, the chunked forward for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc): a file-scope device array of fixed
// size (gdn2.h, GDN2_NOALLOC_SCRATCH_BYTES) that every GPU the library runs
// on holds until the process ends.
//
// The array's host-side name is only a stand-in for the symbol: its device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and only that address is handed to the kernels.
#include "gdn2.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn2_launch.hpp"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[GDN2_NOALLOC_SCRATCH_BYTES];

std::mutex g_lock;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace gdn2 {

void* noalloc_scratch()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> g(g_lock);
    if (g_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace gdn2
