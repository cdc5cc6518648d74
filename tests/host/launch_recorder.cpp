// Recording stand-ins for the kernel launchers of gg_kernels.hip: the host
// driver checks which launches a call makes and with which parameters,
// without a GPU.  Test infrastructure only.
#include "launch_recorder.h"

#include "gg.h"

std::vector<Launch> g_launches;

namespace gg {
static hipError_t rec(const char* kind, const GemmParams& p, int num_cu) {
    g_launches.push_back(Launch{kind, p, num_cu, nullptr, nullptr, 0, 0, 0});
    return hipSuccess;
}
hipError_t launch_fc1_swiglu(const GemmParams& p, int num_cu, hipStream_t) { return rec("fc1_swiglu", p, num_cu); }
hipError_t launch_fc2(const GemmParams& p, int num_cu, hipStream_t) { return rec("fc2", p, num_cu); }
hipError_t launch_dgrad_fc2(const GemmParams& p, int num_cu, hipStream_t) { return rec("dgrad_fc2", p, num_cu); }
hipError_t launch_dgrad_fc1(const GemmParams& p, int num_cu, hipStream_t) { return rec("dgrad_fc1", p, num_cu); }
hipError_t launch_pack_frag(const uint16_t* packed, uint16_t* frag, int E, int H, int F, hipStream_t) {
    Launch l{"pack_frag", GemmParams{}, 0, packed, frag, E, H, F};
    g_launches.push_back(l);
    return hipSuccess;
}
hipError_t launch_round_bf16(const float*, uint16_t*, int64_t n, hipStream_t) {
    Launch l{"round_bf16", GemmParams{}, 0, nullptr, nullptr, static_cast<int>(n), 0, 0};
    g_launches.push_back(l);
    return hipSuccess;
}
hipError_t launch_dp_reduce(const int64_t*, int E, int M, const float*, int ld, float*, hipStream_t) {
    Launch l{"dp_reduce", GemmParams{}, 0, nullptr, nullptr, E, M, ld};
    g_launches.push_back(l);
    return hipSuccess;
}
hipError_t launch_scale_rows(const uint16_t*, const float*, int64_t M, int H, uint16_t*, hipStream_t) {
    Launch l{"scale_rows", GemmParams{}, 0, nullptr, nullptr, static_cast<int>(M), H, 0};
    g_launches.push_back(l);
    return hipSuccess;
}
hipError_t launch_scale_rows_bwd(const uint16_t*, const uint16_t*, const float*, int64_t M, int H, uint16_t*,
                                 float* dprobs, hipStream_t) {
    Launch l{"scale_rows_bwd", GemmParams{}, 0, nullptr, nullptr, static_cast<int>(M), H, dprobs != nullptr};
    g_launches.push_back(l);
    return hipSuccess;
}
// The static scratch array of the no-allocation entry point: one host buffer
// per device here.
hipError_t noalloc_scratch(int device, void** ptr) {
    static std::vector<std::vector<uint8_t>> bufs(8);
    if (device < 0 || device >= 8) return hipErrorInvalidDevice;
    if (bufs[device].empty()) bufs[device].resize(GG_NOALLOC_SCRATCH_BYTES);
    *ptr = bufs[device].data();
    return hipSuccess;
}
}  // namespace gg
