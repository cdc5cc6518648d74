// C-ABI entry points of libgg: argument validation, device checks and
// kernel launches.  Declarations and the contract are in include/gg.h.
//
// Every argument check runs before the first HIP call, so a bad call is
// rejected on any machine, with or without a GPU.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "gg.h"
#include "gg_kernels.h"

static_assert(GG_MAX_EXPERTS == GG_KMAX_EXPERTS, "expert limit mismatch");

namespace {

struct DeviceInfo {
    int checked = 0;      // 0 unknown, 1 gfx950, -1 other
    int num_cu = 0;
    int device = 0;       // device index
};

constexpr int kMaxDevices = 64;
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

// Properties of the device the work will run on: the stream's device, or the
// current device for the null stream.
int device_info(hipStream_t stream, DeviceInfo* out) {
    int dev = 0;
    if (stream == nullptr) {
        if (hipGetDevice(&dev) != hipSuccess) return GG_ERR_HIP;
    } else {
        hipDevice_t d = 0;
        if (hipStreamGetDevice(stream, &d) != hipSuccess) return GG_ERR_HIP;
        dev = static_cast<int>(d);
    }
    if (dev < 0 || dev >= kMaxDevices) return GG_ERR_UNSUPPORTED_DEVICE;
    std::lock_guard<std::mutex> lock(g_dev_mu);
    DeviceInfo& d = g_dev[dev];
    if (d.checked == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GG_ERR_HIP;
        const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        d.num_cu = prop.multiProcessorCount;
        d.device = dev;
        d.checked = ok ? 1 : -1;
    }
    if (d.checked != 1) return GG_ERR_UNSUPPORTED_DEVICE;
    *out = d;
    return GG_OK;
}

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
}

bool overlap(Range a, Range b) {
    return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks common to the GEMM calls.
int check_shape(int64_t M, int64_t E, int64_t H, int64_t F) {
    if (E < 1 || E > GG_MAX_EXPERTS) return GG_ERR_INVALID_ARGUMENT;
    if (H <= 0 || F <= 0 || (H % 8) != 0 || (F % 8) != 0) return GG_ERR_INVALID_ARGUMENT;
    // the kernels address one expert's weight matrix and a 256-row token panel
    // with 32-bit byte offsets
    if (H >= (int64_t(1) << 22) || 2 * F >= (int64_t(1) << 22)) return GG_ERR_INVALID_ARGUMENT;
    if (4 * F * H >= (int64_t(1) << 31)) return GG_ERR_INVALID_ARGUMENT;
    if (M < 0 || M >= (int64_t(1) << 31)) return GG_ERR_INVALID_ARGUMENT;
    return GG_OK;
}

// Outputs must not overlap any input nor each other.
int check_aliasing(const std::vector<Range>& ins, const std::vector<Range>& outs) {
    for (size_t i = 0; i < outs.size(); ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return GG_ERR_ALIASING;
        for (size_t j = i + 1; j < outs.size(); ++j)
            if (overlap(outs[i], outs[j])) return GG_ERR_ALIASING;
    }
    return GG_OK;
}

// Optional synchronous check of the device offsets (GG_DEBUG_VALIDATE=1, read
// at every call so that a process can switch it on and off).
int debug_validate_offsets(const int64_t* offsets, int64_t E, int64_t M, hipStream_t stream) {
    const char* v = std::getenv("GG_DEBUG_VALIDATE");
    if (!(v && v[0] == '1')) return GG_OK;
    std::vector<int64_t> h(static_cast<size_t>(E + 1));
    if (hipMemcpyAsync(h.data(), offsets, sizeof(int64_t) * (E + 1), hipMemcpyDeviceToHost, stream) !=
            hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return GG_ERR_HIP;
    if (h[0] < 0 || h[static_cast<size_t>(E)] > M) return GG_ERR_INVALID_ARGUMENT;
    for (int64_t e = 0; e < E; ++e)
        if (h[e + 1] < h[e]) return GG_ERR_INVALID_ARGUMENT;
    return GG_OK;
}

// Shapes that have fragment-ordered copies (W1, W2, W1^T, W2^T, read by the
// four-wave tiles of FC1, FC2, dX and dA).
bool has_frag(int64_t H, int64_t F) { return H % 256 == 0 && F % 128 == 0; }
// Elements of one expert block of the packed buffer, and of the fragment buffer.
int64_t expert_block(int64_t H, int64_t F) { return 3 * F * H; }
int64_t frag_block(int64_t H, int64_t F) { return gg::FRAG_BLOCK_FH * F * H; }

// Checks of an optional fragment buffer: null (no copies), or a 16-byte
// aligned buffer for a shape that has them.
int check_frag(const void* frag, int64_t H, int64_t F) {
    if (!frag) return GG_OK;
    if (!has_frag(H, F)) return GG_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(frag) & 15u) != 0) return GG_ERR_MISALIGNED;
    return GG_OK;
}

// This GEMM's matrix in the fragment buffer (offset in units of F * H), or null.
const uint16_t* frag_matrix(const void* frag, int which, int64_t H, int64_t F) {
    return frag ? static_cast<const uint16_t*>(frag) + static_cast<int64_t>(which) * F * H : nullptr;
}

gg::GemmParams base_params(const int64_t* offsets, int64_t M, const void* packed, int64_t E,
                           int64_t H, int64_t F) {
    gg::GemmParams p{};
    p.offsets = offsets;
    p.M = static_cast<int>(M);
    p.E = static_cast<int>(E);
    p.w_expert_stride = expert_block(H, F);
    p.w = static_cast<const uint16_t*>(packed);
    p.wfrag_stride = frag_block(H, F);
    p.up_off = static_cast<int>(F);
    p.slope = 1.0f;
    return p;
}

// Slope of the gate activation's sigmoid, or 0 for an unknown activation.
float act_slope(int activation) {
    switch (activation) {
        case GG_ACT_SWIGLU: return 1.0f;
        case GG_ACT_QGEGLU: return 1.702f;
        default: return 0.0f;
    }
}

int64_t dp_groups(int64_t F) { return (F + 31) / 32; }

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

extern "C" {

const char* gg_status_string(int status) {
    switch (status) {
        case GG_OK: return "GG_OK";
        case GG_ERR_INVALID_ARGUMENT: return "GG_ERR_INVALID_ARGUMENT";
        case GG_ERR_MISALIGNED: return "GG_ERR_MISALIGNED";
        case GG_ERR_UNSUPPORTED_DEVICE: return "GG_ERR_UNSUPPORTED_DEVICE (gfx950 required)";
        case GG_ERR_WORKSPACE_TOO_SMALL: return "GG_ERR_WORKSPACE_TOO_SMALL";
        case GG_ERR_ALIASING: return "GG_ERR_ALIASING";
        case GG_ERR_HIP: return "GG_ERR_HIP";
        default: return "unknown gg_status";
    }
}

size_t gg_packed_bytes(int64_t E, int64_t H, int64_t F) {
    if (E <= 0 || H <= 0 || F <= 0) return 0;
    return static_cast<size_t>(2) * static_cast<size_t>(E) * static_cast<size_t>(expert_block(H, F));
}

size_t gg_dgrad_workspace_bytes(int64_t M, int64_t F) {
    if (M <= 0 || F <= 0) return 0;
    return static_cast<size_t>(4) * static_cast<size_t>(M) * static_cast<size_t>(F);
}

size_t gg_dgrad_glu_workspace_bytes(int64_t M, int64_t F, int with_dprobs) {
    if (M <= 0 || F <= 0) return 0;
    size_t n = gg_dgrad_workspace_bytes(M, F);
    if (with_dprobs) n += static_cast<size_t>(4) * static_cast<size_t>(M) * static_cast<size_t>(dp_groups(F));
    return n;
}

size_t gg_frag_bytes(int64_t E, int64_t H, int64_t F) {
    if (E <= 0 || H <= 0 || F <= 0 || !has_frag(H, F)) return 0;
    return static_cast<size_t>(2) * static_cast<size_t>(E) * static_cast<size_t>(frag_block(H, F));
}

int gg_pack_weights(int64_t E, int64_t H, int64_t F, const void* const* w1, const void* const* w2,
                    void* packed, size_t packed_bytes, hipStream_t stream) {
    if (E < 1 || E > GG_MAX_EXPERTS || H <= 0 || F <= 0 || (H % 8) || (F % 8))
        return GG_ERR_INVALID_ARGUMENT;
    if (!w1 || !w2 || !packed) return GG_ERR_INVALID_ARGUMENT;
    if (!aligned16(packed)) return GG_ERR_MISALIGNED;
    const size_t need = gg_packed_bytes(E, H, F);
    if (packed_bytes < need) return GG_ERR_WORKSPACE_TOO_SMALL;
    const size_t w1_bytes = static_cast<size_t>(2 * F * H) * 2;
    const size_t w2_bytes = static_cast<size_t>(H * F) * 2;
    const size_t per_expert = static_cast<size_t>(expert_block(H, F)) * 2;
    const Range whole = range_of(packed, need);
    char* base = static_cast<char*>(packed);
    for (int64_t e = 0; e < E; ++e) {
        if (!w1[e] || !w2[e]) return GG_ERR_INVALID_ARGUMENT;
        if ((reinterpret_cast<uintptr_t>(w1[e]) | reinterpret_cast<uintptr_t>(w2[e])) & 1u)
            return GG_ERR_MISALIGNED;
        const void* d1 = base + e * per_expert;
        const void* d2 = base + e * per_expert + w1_bytes;
        if (w1[e] != d1 && overlap(range_of(w1[e], w1_bytes), whole)) return GG_ERR_ALIASING;
        if (w2[e] != d2 && overlap(range_of(w2[e], w2_bytes), whole)) return GG_ERR_ALIASING;
    }
    DeviceInfo info;
    const int st = device_info(stream, &info);
    if (st != GG_OK) return st;
    for (int64_t e = 0; e < E; ++e) {
        void* d1 = base + e * per_expert;
        void* d2 = base + e * per_expert + w1_bytes;
        if (w1[e] != d1 &&
            hipMemcpyAsync(d1, w1[e], w1_bytes, hipMemcpyDeviceToDevice, stream) != hipSuccess)
            return GG_ERR_HIP;
        if (w2[e] != d2 &&
            hipMemcpyAsync(d2, w2[e], w2_bytes, hipMemcpyDeviceToDevice, stream) != hipSuccess)
            return GG_ERR_HIP;
    }
    return GG_OK;
}

int gg_pack_frag(int64_t E, int64_t H, int64_t F, const void* packed, size_t packed_bytes, void* frag,
                 size_t frag_bytes, hipStream_t stream) {
    if (E < 1 || E > GG_MAX_EXPERTS || H <= 0 || F <= 0 || (H % 8) || (F % 8) || !has_frag(H, F))
        return GG_ERR_INVALID_ARGUMENT;
    if (!packed || !frag) return GG_ERR_INVALID_ARGUMENT;
    if (!aligned16(packed) || !aligned16(frag)) return GG_ERR_MISALIGNED;
    if (packed_bytes < gg_packed_bytes(E, H, F) || frag_bytes < gg_frag_bytes(E, H, F))
        return GG_ERR_WORKSPACE_TOO_SMALL;
    if (overlap(range_of(packed, gg_packed_bytes(E, H, F)), range_of(frag, gg_frag_bytes(E, H, F))))
        return GG_ERR_ALIASING;
    DeviceInfo info;
    const int st = device_info(stream, &info);
    if (st != GG_OK) return st;
    return gg::launch_pack_frag(static_cast<const uint16_t*>(packed), static_cast<uint16_t*>(frag),
                                static_cast<int>(E), static_cast<int>(H), static_cast<int>(F), stream) == hipSuccess
               ? GG_OK
               : GG_ERR_HIP;
}

int gg_forward_fc1_swiglu(const void* x, const int64_t* offsets, int64_t M, const void* packed,
                          int64_t E, int64_t H, int64_t F, void* h1_out, void* a_out,
                          hipStream_t stream) {
    return gg_forward_fc1_glu(x, offsets, M, packed, nullptr, E, H, F, GG_ACT_SWIGLU, nullptr, h1_out, a_out,
                              stream);
}

int gg_forward_fc1_glu(const void* x, const int64_t* offsets, int64_t M, const void* packed, const void* frag,
                       int64_t E, int64_t H, int64_t F, int activation, const float* probs, void* h1_out,
                       void* a_out, hipStream_t stream) {
    int st = check_shape(M, E, H, F);
    if (st != GG_OK) return st;
    const float slope = act_slope(activation);
    if (slope == 0.0f) return GG_ERR_INVALID_ARGUMENT;
    if ((st = check_frag(frag, H, F)) != GG_OK) return st;
    if (M == 0) return GG_OK;
    if (!x || !offsets || !packed || !a_out) return GG_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(packed) || !aligned16(a_out) || (h1_out && !aligned16(h1_out)) ||
        (reinterpret_cast<uintptr_t>(offsets) & 7u) || (probs && !aligned4(probs)))
        return GG_ERR_MISALIGNED;
    std::vector<Range> ins = {range_of(x, M * H * 2), range_of(packed, gg_packed_bytes(E, H, F)),
                              range_of(offsets, (E + 1) * 8)};
    if (probs) ins.push_back(range_of(probs, M * 4));
    if (frag) ins.push_back(range_of(frag, gg_frag_bytes(E, H, F)));
    std::vector<Range> outs = {range_of(a_out, M * F * 2)};
    if (h1_out) outs.push_back(range_of(h1_out, M * 2 * F * 2));
    if ((st = check_aliasing(ins, outs)) != GG_OK) return st;
    DeviceInfo info;
    if ((st = device_info(stream, &info)) != GG_OK) return st;
    if ((st = debug_validate_offsets(offsets, E, M, stream)) != GG_OK) return st;
    gg::GemmParams p = base_params(offsets, M, packed, E, H, F);
    p.act = static_cast<const uint16_t*>(x);
    p.K = static_cast<int>(H);
    p.N = static_cast<int>(F);
    p.ldw = static_cast<int>(H);
    p.out0 = static_cast<uint16_t*>(a_out);
    p.out1 = static_cast<uint16_t*>(h1_out);
    p.slope = slope;
    p.probs = probs;
    p.wfrag = frag_matrix(frag, gg::FRAG_W1, H, F);
    return gg::launch_fc1_swiglu(p, info.num_cu, stream) == hipSuccess ? GG_OK : GG_ERR_HIP;
}

int gg_forward_fc2(const void* a, const int64_t* offsets, int64_t M, const void* packed, int64_t E,
                   int64_t H, int64_t F, void* y, hipStream_t stream) {
    return gg_forward_fc2_frag(a, offsets, M, packed, nullptr, E, H, F, y, stream);
}

int gg_forward_fc2_frag(const void* a, const int64_t* offsets, int64_t M, const void* packed, const void* frag,
                        int64_t E, int64_t H, int64_t F, void* y, hipStream_t stream) {
    int st = check_shape(M, E, H, F);
    if (st != GG_OK) return st;
    if ((st = check_frag(frag, H, F)) != GG_OK) return st;
    if (M == 0) return GG_OK;
    if (!a || !offsets || !packed || !y) return GG_ERR_INVALID_ARGUMENT;
    if (!aligned16(a) || !aligned16(packed) || !aligned16(y) || (reinterpret_cast<uintptr_t>(offsets) & 7u))
        return GG_ERR_MISALIGNED;
    std::vector<Range> ins = {range_of(a, M * F * 2), range_of(packed, gg_packed_bytes(E, H, F)),
                              range_of(offsets, (E + 1) * 8)};
    if (frag) ins.push_back(range_of(frag, gg_frag_bytes(E, H, F)));
    std::vector<Range> outs = {range_of(y, M * H * 2)};
    if ((st = check_aliasing(ins, outs)) != GG_OK) return st;
    DeviceInfo info;
    if ((st = device_info(stream, &info)) != GG_OK) return st;
    if ((st = debug_validate_offsets(offsets, E, M, stream)) != GG_OK) return st;
    gg::GemmParams p = base_params(offsets, M, packed, E, H, F);
    p.w = static_cast<const uint16_t*>(packed) + 2 * F * H;
    p.act = static_cast<const uint16_t*>(a);
    p.K = static_cast<int>(F);
    p.N = static_cast<int>(H);
    p.ldw = static_cast<int>(F);
    p.out0 = static_cast<uint16_t*>(y);
    p.wfrag = frag_matrix(frag, gg::FRAG_W2, H, F);
    return gg::launch_fc2(p, info.num_cu, stream) == hipSuccess ? GG_OK : GG_ERR_HIP;
}

int gg_dgrad(const void* dy, const void* h1, const int64_t* offsets, int64_t M, const void* packed,
             int64_t E, int64_t H, int64_t F, void* workspace, size_t workspace_bytes, void* dx,
             hipStream_t stream) {
    return gg_dgrad_glu(dy, h1, offsets, M, packed, nullptr, E, H, F, GG_ACT_SWIGLU, nullptr, workspace,
                        workspace_bytes, dx, nullptr, stream);
}

}  // extern "C"

namespace {

// Input gradient from the saved H1 (h1 != null) or from X, recomputing H1 into
// the workspace first (x != null; exactly one of the two is given).
int dgrad_impl(const void* dy, const void* h1, const void* x, const int64_t* offsets, int64_t M,
               const void* packed, const void* frag, int64_t E, int64_t H, int64_t F, int activation,
               const float* probs, void* workspace, size_t workspace_bytes, void* dx, float* dprobs,
               hipStream_t stream) {
    int st = check_shape(M, E, H, F);
    if (st != GG_OK) return st;
    const float slope = act_slope(activation);
    if (slope == 0.0f) return GG_ERR_INVALID_ARGUMENT;
    if ((st = check_frag(frag, H, F)) != GG_OK) return st;
    if (M == 0) return GG_OK;
    const void* src = h1 ? h1 : x;   // the saved H1 [M][2F], or X [M][H]
    if (!dy || !src || !offsets || !packed || !workspace || !dx) return GG_ERR_INVALID_ARGUMENT;
    if (!aligned16(dy) || !aligned16(src) || !aligned16(packed) || !aligned16(workspace) ||
        !aligned16(dx) || (reinterpret_cast<uintptr_t>(offsets) & 7u) || (probs && !aligned4(probs)) ||
        (dprobs && !aligned4(dprobs)))
        return GG_ERR_MISALIGNED;
    const size_t ws_need = gg_dgrad_glu_workspace_bytes(M, F, dprobs != nullptr);
    if (workspace_bytes < ws_need) return GG_ERR_WORKSPACE_TOO_SMALL;
    std::vector<Range> ins = {range_of(dy, M * H * 2), range_of(src, h1 ? M * 2 * F * 2 : M * H * 2),
                              range_of(packed, gg_packed_bytes(E, H, F)), range_of(offsets, (E + 1) * 8)};
    if (probs) ins.push_back(range_of(probs, M * 4));
    if (frag) ins.push_back(range_of(frag, gg_frag_bytes(E, H, F)));
    std::vector<Range> outs = {range_of(workspace, ws_need), range_of(dx, M * H * 2)};
    if (dprobs) outs.push_back(range_of(dprobs, M * 4));
    if ((st = check_aliasing(ins, outs)) != GG_OK) return st;
    DeviceInfo info;
    if ((st = device_info(stream, &info)) != GG_OK) return st;
    if ((st = debug_validate_offsets(offsets, E, M, stream)) != GG_OK) return st;
    if (!h1) {
        // recompute H1 = X W1_e^T into the workspace: FC1 as a plain GEMM over
        // W1's 2F rows (gate | up), the same sums the forward rounds
        gg::GemmParams r = base_params(offsets, M, packed, E, H, F);
        r.act = static_cast<const uint16_t*>(x);
        r.K = static_cast<int>(H);
        r.N = static_cast<int>(2 * F);
        r.ldw = static_cast<int>(H);
        r.out0 = static_cast<uint16_t*>(workspace);
        if (frag) {   // the four-wave kernel over W1's fragment copy, columns put back in H1 order
            r.wfrag = frag_matrix(frag, gg::FRAG_W1, H, F);
            r.h1_order = 1;
        }
        if (gg::launch_fc2(r, info.num_cu, stream) != hipSuccess) return GG_ERR_HIP;
    }
    // dA = dY W2_e, then the activation derivative with H1 -> dH1 (workspace;
    // with a recomputed H1 in place: each H1 element is read only by the lane
    // that then writes the dH1 element at the same position)
    gg::GemmParams p = base_params(offsets, M, packed, E, H, F);
    p.w = static_cast<const uint16_t*>(packed) + 2 * F * H;
    p.act = static_cast<const uint16_t*>(dy);
    p.K = static_cast<int>(H);
    p.N = static_cast<int>(F);
    p.ldw = static_cast<int>(F);
    p.aux = h1 ? static_cast<const uint16_t*>(h1) : static_cast<const uint16_t*>(workspace);
    p.out0 = static_cast<uint16_t*>(workspace);
    p.slope = slope;
    p.probs = probs;
    // dp partial sums [M][ceil(F/32)] fp32 after dH1 in the workspace
    float* dp_part = dprobs ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                       gg_dgrad_workspace_bytes(M, F))
                            : nullptr;
    p.dp_part = dp_part;
    p.dp_ld = static_cast<int>(dp_groups(F));
    p.wfrag = frag_matrix(frag, gg::FRAG_W2T, H, F);   // W2^T fragments (four-wave tiles, F % 256 == 0)
    if (gg::launch_dgrad_fc2(p, info.num_cu, stream) != hipSuccess) return GG_ERR_HIP;
    if (dprobs && gg::launch_dp_reduce(offsets, static_cast<int>(E), static_cast<int>(M), dp_part,
                                       static_cast<int>(dp_groups(F)), dprobs, stream) != hipSuccess)
        return GG_ERR_HIP;
    // dX = dH1 W1_e
    gg::GemmParams q = base_params(offsets, M, packed, E, H, F);
    q.act = static_cast<const uint16_t*>(workspace);
    q.K = static_cast<int>(2 * F);
    q.N = static_cast<int>(H);
    q.ldw = static_cast<int>(H);
    q.out0 = static_cast<uint16_t*>(dx);
    q.wfrag = frag_matrix(frag, gg::FRAG_W1T, H, F);   // W1^T fragments: the same K-contiguous form
    return gg::launch_dgrad_fc1(q, info.num_cu, stream) == hipSuccess ? GG_OK : GG_ERR_HIP;
}

}  // namespace

extern "C" {

int gg_dgrad_glu(const void* dy, const void* h1, const int64_t* offsets, int64_t M, const void* packed,
                 const void* frag, int64_t E, int64_t H, int64_t F, int activation, const float* probs,
                 void* workspace, size_t workspace_bytes, void* dx, float* dprobs, hipStream_t stream) {
    if (M > 0 && !h1) return GG_ERR_INVALID_ARGUMENT;
    return dgrad_impl(dy, h1, nullptr, offsets, M, packed, frag, E, H, F, activation, probs, workspace,
                      workspace_bytes, dx, dprobs, stream);
}

int gg_dgrad_recompute(const void* dy, const void* x, const int64_t* offsets, int64_t M, const void* packed,
                       const void* frag, int64_t E, int64_t H, int64_t F, int activation, const float* probs,
                       void* workspace, size_t workspace_bytes, void* dx, float* dprobs, hipStream_t stream) {
    if (M > 0 && !x) return GG_ERR_INVALID_ARGUMENT;
    return dgrad_impl(dy, nullptr, x, offsets, M, packed, frag, E, H, F, activation, probs, workspace,
                      workspace_bytes, dx, dprobs, stream);
}

int gg_dgrad_noalloc(const void* dy, const void* h1, const int64_t* offsets, int64_t M, const void* packed,
                     int64_t E, int64_t H, int64_t F, void* dx, hipStream_t stream) {
    int st = check_shape(M, E, H, F);
    if (st != GG_OK) return st;
    if (M == 0) return GG_OK;
    if (gg_dgrad_workspace_bytes(M, F) > static_cast<size_t>(GG_NOALLOC_SCRATCH_BYTES))
        return GG_ERR_WORKSPACE_TOO_SMALL;
    if (!dy || !h1 || !offsets || !packed || !dx) return GG_ERR_INVALID_ARGUMENT;
    DeviceInfo info;
    if ((st = device_info(stream, &info)) != GG_OK) return st;
    // dH1 goes to this device's copy of the static scratch array
    void* scratch = nullptr;
    if (gg::noalloc_scratch(info.device, &scratch) != hipSuccess) return GG_ERR_HIP;
    return dgrad_impl(dy, h1, nullptr, offsets, M, packed, nullptr, E, H, F, GG_ACT_SWIGLU, nullptr, scratch,
                      static_cast<size_t>(GG_NOALLOC_SCRATCH_BYTES), dx, nullptr, stream);
}

int gg_scale_rows(const void* x, const float* probs, int64_t M, int64_t H, void* x_out, hipStream_t stream) {
    if (M < 0 || M >= (int64_t(1) << 31) || H <= 0 || H % 8 != 0 || H >= (int64_t(1) << 22))
        return GG_ERR_INVALID_ARGUMENT;
    if (M == 0) return GG_OK;
    if (!x || !probs || !x_out) return GG_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(x_out) || !aligned4(probs)) return GG_ERR_MISALIGNED;
    const size_t xb = static_cast<size_t>(M * H) * 2;
    const Range out = range_of(x_out, xb);
    if ((x != x_out && overlap(out, range_of(x, xb))) || overlap(out, range_of(probs, M * 4)))
        return GG_ERR_ALIASING;
    DeviceInfo info;
    const int st = device_info(stream, &info);
    if (st != GG_OK) return st;
    return gg::launch_scale_rows(static_cast<const uint16_t*>(x), probs, M, static_cast<int>(H),
                                 static_cast<uint16_t*>(x_out), stream) == hipSuccess
               ? GG_OK
               : GG_ERR_HIP;
}

int gg_scale_rows_backward(const void* dxs, const void* x, const float* probs, int64_t M, int64_t H, void* dx,
                           float* dprobs, hipStream_t stream) {
    if (M < 0 || M >= (int64_t(1) << 31) || H <= 0 || H % 8 != 0 || H >= (int64_t(1) << 22))
        return GG_ERR_INVALID_ARGUMENT;
    if (M == 0) return GG_OK;
    if (!dxs || !x || !probs || !dx) return GG_ERR_INVALID_ARGUMENT;
    if (!aligned16(dxs) || !aligned16(x) || !aligned16(dx) || !aligned4(probs) || (dprobs && !aligned4(dprobs)))
        return GG_ERR_MISALIGNED;
    const size_t xb = static_cast<size_t>(M * H) * 2;
    const Range rdx = range_of(dx, xb), rx = range_of(x, xb), rp = range_of(probs, M * 4);
    const Range rdp = dprobs ? range_of(dprobs, M * 4) : Range{0, 0};
    // dx may be dxs itself; nothing else may overlap an output
    if ((dx != dxs && overlap(rdx, range_of(dxs, xb))) || overlap(rdx, rx) || overlap(rdx, rp) ||
        overlap(rdp, range_of(dxs, xb)) || overlap(rdp, rx) || overlap(rdp, rp) || overlap(rdp, rdx))
        return GG_ERR_ALIASING;
    DeviceInfo info;
    const int st = device_info(stream, &info);
    if (st != GG_OK) return st;
    return gg::launch_scale_rows_bwd(static_cast<const uint16_t*>(dxs), static_cast<const uint16_t*>(x), probs, M,
                                     static_cast<int>(H), static_cast<uint16_t*>(dx), dprobs, stream) == hipSuccess
               ? GG_OK
               : GG_ERR_HIP;
}

int gg_round_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t stream) {
    if (n < 0) return GG_ERR_INVALID_ARGUMENT;
    if (n == 0) return GG_OK;
    if (!in || !out) return GG_ERR_INVALID_ARGUMENT;
    if (overlap(range_of(in, n * 4), range_of(out, n * 2))) return GG_ERR_ALIASING;
    DeviceInfo info;
    const int st = device_info(stream, &info);
    if (st != GG_OK) return st;
    return gg::launch_round_bf16(in, out, n, stream) == hipSuccess ? GG_OK : GG_ERR_HIP;
}

}  // extern "C"
