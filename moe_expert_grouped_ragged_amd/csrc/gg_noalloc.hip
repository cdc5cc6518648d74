// Device-resident scratch for the entry point that allocates nothing
// (gg_dgrad_noalloc): a file-scope device array, one copy per GPU, held
// until the process ends.  Host code never passes the array's name to a
// kernel or a copy (on the host it is only a stand-in symbol): each device's
// address is looked up once, with that device current, and cached here.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gg.h"
#include "gg_kernels.h"

namespace {

static __device__ __align__(256) uint8_t scratch[GG_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

}  // namespace

namespace gg {

hipError_t noalloc_scratch(int device, void** ptr) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        int current = 0;
        hipError_t st = hipGetDevice(&current);
        if (st != hipSuccess) return st;
        if (current != device && (st = hipSetDevice(device)) != hipSuccess) return st;
        void* p = nullptr;
        st = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = current != device ? hipSetDevice(current) : hipSuccess;
        if (st != hipSuccess) return st;
        if (back != hipSuccess) return back;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = p;
    }
    *ptr = g_scratch_ptr[device];
    return hipSuccess;
}

}  // namespace gg
