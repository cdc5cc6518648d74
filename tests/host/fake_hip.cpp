// A stand-in for the five HIP runtime calls the C-ABI layer makes, so that
// gg_api.cpp can be built and driven on a machine without a GPU (under the
// address and undefined-behaviour sanitizers).  "Device" memory is host
// memory here.  A stream handle encodes its device: (device + 1) << 4; the
// null stream means the current device.  Test infrastructure only.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstring>

#include "fake_hip.h"

namespace {
char g_arch[8][32] = {"gfx950", "gfx950", "gfx950", "gfx950", "gfx950", "gfx950", "gfx950", "gfx950"};
int g_current = 0;
int g_fail = 0;
long g_sync_calls = 0, g_d2h_calls = 0, g_d2d_calls = 0, g_prop_calls = 0;
}  // namespace

void fake_set_arch(int dev, const char* arch) { std::strncpy(g_arch[dev], arch, sizeof(g_arch[dev]) - 1); }
void fake_set_current(int dev) { g_current = dev; }
void fake_set_fail(int fail) { g_fail = fail; }
hipStream_t fake_stream(int dev) { return reinterpret_cast<hipStream_t>(static_cast<uintptr_t>(dev + 1) << 4); }
long fake_count(const char* what) {
    if (!std::strcmp(what, "sync")) return g_sync_calls;
    if (!std::strcmp(what, "d2h")) return g_d2h_calls;
    if (!std::strcmp(what, "d2d")) return g_d2d_calls;
    if (!std::strcmp(what, "prop")) return g_prop_calls;
    return -1;
}

hipError_t hipGetDevice(int* device) {
    if (g_fail) return hipErrorNoDevice;
    *device = g_current;
    return hipSuccess;
}

hipError_t hipStreamGetDevice(hipStream_t stream, hipDevice_t* device) {
    if (g_fail) return hipErrorNoDevice;
    const uintptr_t v = reinterpret_cast<uintptr_t>(stream);
    if (v == 0 || (v & 15u) != 0 || (v >> 4) > 8) return hipErrorInvalidHandle;
    *device = static_cast<hipDevice_t>((v >> 4) - 1);
    return hipSuccess;
}

hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* prop, int device) {
    if (g_fail || device < 0 || device >= 8) return hipErrorInvalidDevice;
    ++g_prop_calls;
    std::memset(prop, 0, sizeof(*prop));
    std::strncpy(prop->gcnArchName, g_arch[device], sizeof(prop->gcnArchName) - 1);
    prop->multiProcessorCount = 256;
    return hipSuccess;
}

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind kind, hipStream_t) {
    if (g_fail) return hipErrorNoDevice;
    if (kind == hipMemcpyDeviceToHost) ++g_d2h_calls;
    if (kind == hipMemcpyDeviceToDevice) ++g_d2d_calls;
    std::memmove(dst, src, bytes);
    return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t) {
    ++g_sync_calls;
    return g_fail ? hipErrorNoDevice : hipSuccess;
}
