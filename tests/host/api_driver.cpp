// Host-side driver of the C-ABI layer (gg_api.cpp) built with the fake HIP
// runtime and the recording launchers: argument checks, the launches each
// entry point makes and their parameters, device checks, the debug offset
// check and the packing copies.  Built and run under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitized.py.  Exit status 0
// when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "fake_hip.h"
#include "gg.h"
#include "launch_recorder.h"

static int g_failed = 0, g_checked = 0;
#define CHECK(cond)                                                              \
    do {                                                                         \
        ++g_checked;                                                             \
        if (!(cond)) {                                                           \
            ++g_failed;                                                          \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
        }                                                                        \
    } while (0)

// 16-byte aligned host buffers standing in for device memory.
struct Buf {
    std::vector<uint8_t> raw;
    uint8_t* p;
    explicit Buf(size_t n) : raw(n + 64, 0) {
        p = raw.data() + ((16 - (reinterpret_cast<uintptr_t>(raw.data()) & 15)) & 15);
    }
    template <typename T> T* as() { return reinterpret_cast<T*>(p); }
};

static void test_sizes() {
    CHECK(gg_packed_bytes(4, 64, 128) == size_t(6) * 4 * 64 * 128);
    CHECK(gg_packed_bytes(128, 4096, 2048) == size_t(6442450944ull));
    CHECK(gg_packed_bytes(0, 64, 128) == 0 && gg_packed_bytes(4, -8, 128) == 0);
    CHECK(gg_frag_bytes(3, 256, 128) == size_t(12) * 3 * 256 * 128);
    CHECK(gg_frag_bytes(3, 264, 128) == 0 && gg_frag_bytes(3, 256, 136) == 0);
    CHECK(gg_dgrad_workspace_bytes(10, 16) == 640 && gg_dgrad_workspace_bytes(0, 16) == 0);
    CHECK(gg_dgrad_glu_workspace_bytes(10, 40, 1) == 4 * 10 * 40 + 4 * 10 * 2);
    CHECK(std::strcmp(gg_status_string(GG_ERR_ALIASING), "GG_ERR_ALIASING") == 0);
    CHECK(std::strcmp(gg_status_string(99), "unknown gg_status") == 0);
}

static void test_forward_launches() {
    const int64_t E = 3, H = 256, F = 128, M = 40;
    Buf x(M * H * 2), off((E + 1) * 8), pk(gg_packed_bytes(E, H, F)), fr(gg_frag_bytes(E, H, F));
    Buf h1(M * 2 * F * 2), a(M * F * 2), y(M * H * 2);
    hipStream_t s = fake_stream(0);
    g_launches.clear();
    CHECK(gg_forward_fc1_swiglu(x.p, off.as<int64_t>(), M, pk.p, E, H, F, h1.p, a.p, s) == GG_OK);
    CHECK(g_launches.size() == 1 && !std::strcmp(g_launches[0].kind, "fc1_swiglu"));
    const gg::GemmParams& p = g_launches[0].p;
    CHECK(p.K == H && p.N == F && p.ldw == H && p.up_off == F && p.M == M && p.E == E);
    CHECK(p.w == pk.as<uint16_t>() && p.w_expert_stride == 3 * F * H && p.wfrag == nullptr);
    CHECK(p.out0 == a.as<uint16_t>() && p.out1 == h1.as<uint16_t>() && p.slope == 1.0f && !p.probs);
    CHECK(g_launches[0].num_cu == 256);
    // with the fragment buffer: W1's copy at its start, expert stride 6FH
    g_launches.clear();
    CHECK(gg_forward_fc1_glu(x.p, off.as<int64_t>(), M, pk.p, fr.p, E, H, F, GG_ACT_QGEGLU, nullptr, nullptr,
                             a.p, s) == GG_OK);
    CHECK(g_launches.size() == 1 && g_launches[0].p.wfrag == fr.as<uint16_t>());
    CHECK(g_launches[0].p.wfrag_stride == 6 * F * H && g_launches[0].p.slope == 1.702f);
    CHECK(g_launches[0].p.out1 == nullptr);
    // FC2: W2 after W1 in both buffers
    g_launches.clear();
    CHECK(gg_forward_fc2_frag(a.p, off.as<int64_t>(), M, pk.p, fr.p, E, H, F, y.p, s) == GG_OK);
    CHECK(g_launches.size() == 1 && !std::strcmp(g_launches[0].kind, "fc2"));
    CHECK(g_launches[0].p.w == pk.as<uint16_t>() + 2 * F * H && g_launches[0].p.wfrag == fr.as<uint16_t>() + 2 * F * H);
    CHECK(g_launches[0].p.K == F && g_launches[0].p.N == H && g_launches[0].p.ldw == F);
    g_launches.clear();
    CHECK(gg_forward_fc2(a.p, off.as<int64_t>(), M, pk.p, E, H, F, y.p, s) == GG_OK);
    CHECK(g_launches.size() == 1 && g_launches[0].p.wfrag == nullptr);
    // a fragment buffer for a shape without copies
    CHECK(gg_forward_fc2_frag(a.p, off.as<int64_t>(), M, pk.p, fr.p, E, 264, F, y.p, s) == GG_ERR_INVALID_ARGUMENT);
    // M == 0: success and no launch, whatever the pointers
    g_launches.clear();
    CHECK(gg_forward_fc1_swiglu(nullptr, nullptr, 0, nullptr, E, H, F, nullptr, nullptr, s) == GG_OK);
    CHECK(gg_forward_fc2(nullptr, nullptr, 0, nullptr, E, H, F, nullptr, s) == GG_OK);
    CHECK(g_launches.empty());
}

static void test_dgrad_launches() {
    const int64_t E = 2, H = 256, F = 128, M = 33;
    Buf dy(M * H * 2), h1(M * 2 * F * 2), x(M * H * 2), off((E + 1) * 8), pk(gg_packed_bytes(E, H, F));
    Buf fr(gg_frag_bytes(E, H, F)), ws(gg_dgrad_glu_workspace_bytes(M, F, 1)), dx(M * H * 2), dp(M * 4), pr(M * 4);
    hipStream_t s = fake_stream(0);
    g_launches.clear();
    CHECK(gg_dgrad(dy.p, h1.p, off.as<int64_t>(), M, pk.p, E, H, F, ws.p, gg_dgrad_workspace_bytes(M, F), dx.p, s) ==
          GG_OK);
    CHECK(g_launches.size() == 2);
    if (g_launches.size() == 2) {
        const gg::GemmParams& a = g_launches[0].p;
        const gg::GemmParams& b = g_launches[1].p;
        CHECK(!std::strcmp(g_launches[0].kind, "dgrad_fc2") && !std::strcmp(g_launches[1].kind, "dgrad_fc1"));
        CHECK(a.K == H && a.N == F && a.w == pk.as<uint16_t>() + 2 * F * H && a.aux == h1.as<uint16_t>());
        CHECK(a.out0 == ws.as<uint16_t>() && a.dp_part == nullptr);
        CHECK(b.act == ws.as<uint16_t>() && b.K == 2 * F && b.N == H && b.out0 == dx.as<uint16_t>());
        CHECK(b.wfrag == nullptr);
    }
    // with dprobs, probs and the fragment buffer: the dp reduction runs
    // between the two GEMMs, dX reads W1^T's copy
    g_launches.clear();
    CHECK(gg_dgrad_glu(dy.p, h1.p, off.as<int64_t>(), M, pk.p, fr.p, E, H, F, GG_ACT_SWIGLU, pr.as<float>(), ws.p,
                       gg_dgrad_glu_workspace_bytes(M, F, 1), dx.p, dp.as<float>(), s) == GG_OK);
    CHECK(g_launches.size() == 3);
    if (g_launches.size() == 3) {
        CHECK(!std::strcmp(g_launches[1].kind, "dp_reduce") && g_launches[1].c == (F + 31) / 32);
        CHECK(g_launches[0].p.dp_part == reinterpret_cast<float*>(ws.p + gg_dgrad_workspace_bytes(M, F)));
        CHECK(g_launches[2].p.wfrag == fr.as<uint16_t>() + 3 * F * H && g_launches[2].p.wfrag_stride == 6 * F * H);
        CHECK(g_launches[0].p.wfrag == fr.as<uint16_t>() + 5 * F * H);   // W2^T for dA
    }
    // the workspace must hold the partial sums
    CHECK(gg_dgrad_glu(dy.p, h1.p, off.as<int64_t>(), M, pk.p, nullptr, E, H, F, 0, nullptr, ws.p,
                       gg_dgrad_glu_workspace_bytes(M, F, 1) - 4, dx.p, dp.as<float>(), s) == GG_ERR_WORKSPACE_TOO_SMALL);
    // recompute: H1 = X W1^T into the workspace first, over W1's copy in H1 order
    g_launches.clear();
    CHECK(gg_dgrad_recompute(dy.p, x.p, off.as<int64_t>(), M, pk.p, fr.p, E, H, F, 0, nullptr, ws.p,
                             gg_dgrad_workspace_bytes(M, F), dx.p, nullptr, s) == GG_OK);
    CHECK(g_launches.size() == 3);
    if (g_launches.size() == 3) {
        const gg::GemmParams& r = g_launches[0].p;
        CHECK(!std::strcmp(g_launches[0].kind, "fc2") && r.N == 2 * F && r.K == H && r.h1_order == 1);
        CHECK(r.wfrag == fr.as<uint16_t>() && r.out0 == ws.as<uint16_t>());
        CHECK(g_launches[1].p.aux == ws.as<uint16_t>());
    }
    CHECK(gg_dgrad_recompute(dy.p, nullptr, off.as<int64_t>(), M, pk.p, nullptr, E, H, F, 0, nullptr, ws.p,
                             gg_dgrad_workspace_bytes(M, F), dx.p, nullptr, s) == GG_ERR_INVALID_ARGUMENT);
}

static void test_argument_checks() {
    const int64_t E = 2, H = 64, F = 64, M = 8;
    Buf x(M * H * 2), off((E + 1) * 8), pk(gg_packed_bytes(E, H, F)), a(M * F * 2), y(M * H * 2);
    hipStream_t s = fake_stream(0);
    g_launches.clear();
    const long props = fake_count("prop");
    CHECK(gg_forward_fc2(a.p, off.as<int64_t>(), M, pk.p, 0, H, F, y.p, s) == GG_ERR_INVALID_ARGUMENT);
    CHECK(gg_forward_fc2(a.p, off.as<int64_t>(), M, pk.p, GG_MAX_EXPERTS + 1, H, F, y.p, s) == GG_ERR_INVALID_ARGUMENT);
    CHECK(gg_forward_fc2(a.p, off.as<int64_t>(), -1, pk.p, E, H, F, y.p, s) == GG_ERR_INVALID_ARGUMENT);
    CHECK(gg_forward_fc2(a.p, off.as<int64_t>(), M, pk.p, E, 60, F, y.p, s) == GG_ERR_INVALID_ARGUMENT);
    CHECK(gg_forward_fc2(a.p, nullptr, M, pk.p, E, H, F, y.p, s) == GG_ERR_INVALID_ARGUMENT);
    CHECK(gg_forward_fc2(a.p + 2, off.as<int64_t>(), M, pk.p, E, H, F, y.p, s) == GG_ERR_MISALIGNED);
    CHECK(gg_forward_fc2(a.p, reinterpret_cast<int64_t*>(off.p + 4), M, pk.p, E, H, F, y.p, s) == GG_ERR_MISALIGNED);
    CHECK(gg_forward_fc2(a.p, off.as<int64_t>(), M, pk.p, E, H, F, a.p + 16, s) == GG_ERR_ALIASING);
    CHECK(gg_forward_fc2(a.p, off.as<int64_t>(), M, pk.p, E, H, F, pk.p + 64, s) == GG_ERR_ALIASING);
    CHECK(gg_forward_fc1_swiglu(x.p, off.as<int64_t>(), M, pk.p, E, H, F, y.p, y.p + 32, s) == GG_ERR_ALIASING);
    CHECK(gg_forward_fc1_glu(x.p, off.as<int64_t>(), M, pk.p, nullptr, E, H, F, 7, nullptr, nullptr, a.p, s) ==
          GG_ERR_INVALID_ARGUMENT);
    CHECK(gg_round_bf16(nullptr, nullptr, -1, s) == GG_ERR_INVALID_ARGUMENT);
    CHECK(gg_round_bf16(x.as<float>(), reinterpret_cast<uint16_t*>(x.p + 8), 16, s) == GG_ERR_ALIASING);
    // no argument error reached the device or launched anything
    CHECK(g_launches.empty() && fake_count("prop") == props);
}

static void test_devices() {
    const int64_t E = 2, H = 64, F = 64, M = 8;
    Buf off((E + 1) * 8), pk(gg_packed_bytes(E, H, F)), a(M * F * 2), y(M * H * 2), in(64 * 4), out(64 * 2);
    fake_set_arch(3, "gfx942");
    g_launches.clear();
    // the stream's device decides; the null stream means the current device
    CHECK(gg_forward_fc2(a.p, off.as<int64_t>(), M, pk.p, E, H, F, y.p, fake_stream(3)) == GG_ERR_UNSUPPORTED_DEVICE);
    CHECK(gg_round_bf16(in.as<float>(), out.as<uint16_t>(), 64, fake_stream(3)) == GG_ERR_UNSUPPORTED_DEVICE);
    fake_set_current(3);
    CHECK(gg_forward_fc2(a.p, off.as<int64_t>(), M, pk.p, E, H, F, y.p, nullptr) == GG_ERR_UNSUPPORTED_DEVICE);
    fake_set_current(0);
    CHECK(gg_forward_fc2(a.p, off.as<int64_t>(), M, pk.p, E, H, F, y.p, nullptr) == GG_OK);
    CHECK(gg_forward_fc2(a.p, off.as<int64_t>(), M, pk.p, E, H, F, y.p, fake_stream(2)) == GG_OK);
    CHECK(g_launches.size() == 2);
    // the architecture is looked up once per device
    const long props = fake_count("prop");
    CHECK(gg_forward_fc2(a.p, off.as<int64_t>(), M, pk.p, E, H, F, y.p, fake_stream(2)) == GG_OK);
    CHECK(fake_count("prop") == props);
    // a runtime that fails gives GG_ERR_HIP; a bad stream handle too
    fake_set_fail(1);
    CHECK(gg_forward_fc2(a.p, off.as<int64_t>(), M, pk.p, E, H, F, y.p, fake_stream(5)) == GG_ERR_HIP);
    fake_set_fail(0);
    CHECK(gg_forward_fc2(a.p, off.as<int64_t>(), M, pk.p, E, H, F, y.p,
                         reinterpret_cast<hipStream_t>(uintptr_t(12))) == GG_ERR_HIP);
}

static void test_debug_validate() {
    const int64_t E = 3, H = 64, F = 64, M = 16;
    Buf off((E + 1) * 8), pk(gg_packed_bytes(E, H, F)), a(M * F * 2), y(M * H * 2);
    int64_t* o = off.as<int64_t>();
    hipStream_t s = fake_stream(0);
    const int64_t bad[][4] = {{0, 5, 3, 16},      // decreasing
                              {0, 5, 9, 17},      // past M
                              {-1, 5, 9, 16}};    // negative start
    const int64_t good[4] = {0, 5, 5, 16};
    // off: bad offsets are not read on the host (the kernels clamp them)
    unsetenv("GG_DEBUG_VALIDATE");
    std::memcpy(o, bad[0], sizeof(bad[0]));
    g_launches.clear();
    CHECK(gg_forward_fc2(a.p, o, M, pk.p, E, H, F, y.p, s) == GG_OK && g_launches.size() == 1);
    // on: a synchronous check rejects them before any launch
    setenv("GG_DEBUG_VALIDATE", "1", 1);
    for (const auto& b : bad) {
        std::memcpy(o, b, sizeof(b));
        g_launches.clear();
        const long syncs = fake_count("sync");
        CHECK(gg_forward_fc2(a.p, o, M, pk.p, E, H, F, y.p, s) == GG_ERR_INVALID_ARGUMENT);
        CHECK(g_launches.empty() && fake_count("sync") == syncs + 1);
    }
    std::memcpy(o, good, sizeof(good));
    g_launches.clear();
    CHECK(gg_forward_fc2(a.p, o, M, pk.p, E, H, F, y.p, s) == GG_OK && g_launches.size() == 1);
    unsetenv("GG_DEBUG_VALIDATE");
}

static void test_pack() {
    const int64_t E = 3, H = 16, F = 8;
    const size_t w1n = 2 * F * H, w2n = H * F, blk = 3 * F * H;
    std::vector<std::vector<uint16_t>> w1(E, std::vector<uint16_t>(w1n)), w2(E, std::vector<uint16_t>(w2n));
    for (int64_t e = 0; e < E; ++e) {
        for (size_t i = 0; i < w1n; ++i) w1[e][i] = static_cast<uint16_t>(1000 * e + i);
        for (size_t i = 0; i < w2n; ++i) w2[e][i] = static_cast<uint16_t>(30000 + 1000 * e + i);
    }
    Buf pk(gg_packed_bytes(E, H, F));
    const void* s1[3] = {w1[0].data(), w1[1].data(), w1[2].data()};
    const void* s2[3] = {w2[0].data(), w2[1].data(), w2[2].data()};
    hipStream_t s = fake_stream(0);
    long d2d = fake_count("d2d");
    CHECK(gg_pack_weights(E, H, F, s1, s2, pk.p, gg_packed_bytes(E, H, F), s) == GG_OK);
    CHECK(fake_count("d2d") == d2d + 2 * E);
    const uint16_t* P = pk.as<uint16_t>();
    bool layout = true;
    for (int64_t e = 0; e < E; ++e) {
        layout &= std::memcmp(P + e * blk, w1[e].data(), w1n * 2) == 0;
        layout &= std::memcmp(P + e * blk + w1n, w2[e].data(), w2n * 2) == 0;
    }
    CHECK(layout);
    // sources that are their own destinations are skipped: only the replaced
    // middle expert is copied
    std::vector<uint16_t> fresh(w1n, 7);
    const void* v1[3] = {P, fresh.data(), P + 2 * blk};
    const void* v2[3] = {P + w1n, P + blk + w1n, P + 2 * blk + w1n};
    d2d = fake_count("d2d");
    CHECK(gg_pack_weights(E, H, F, v1, v2, pk.p, gg_packed_bytes(E, H, F), s) == GG_OK);
    CHECK(fake_count("d2d") == d2d + 1 && P[blk] == 7 && P[0] == w1[0][0]);
    // partial overlap with the buffer, too small a buffer, misaligned weights
    const void* o1[3] = {P + 8, s1[1], s1[2]};
    CHECK(gg_pack_weights(E, H, F, o1, s2, pk.p, gg_packed_bytes(E, H, F), s) == GG_ERR_ALIASING);
    CHECK(gg_pack_weights(E, H, F, s1, s2, pk.p, gg_packed_bytes(E, H, F) - 2, s) == GG_ERR_WORKSPACE_TOO_SMALL);
    const void* m1[3] = {reinterpret_cast<const uint8_t*>(s1[0]) + 1, s1[1], s1[2]};
    CHECK(gg_pack_weights(E, H, F, m1, s2, pk.p, gg_packed_bytes(E, H, F), s) == GG_ERR_MISALIGNED);
    // the fragment copies: one launch, shapes without copies refused
    const int64_t E2 = 2, H2 = 256, F2 = 128;
    Buf pk2(gg_packed_bytes(E2, H2, F2)), fr2(gg_frag_bytes(E2, H2, F2));
    g_launches.clear();
    CHECK(gg_pack_frag(E2, H2, F2, pk2.p, gg_packed_bytes(E2, H2, F2), fr2.p, gg_frag_bytes(E2, H2, F2), s) == GG_OK);
    CHECK(g_launches.size() == 1 && g_launches[0].frag == fr2.as<uint16_t>() && g_launches[0].a == E2);
    CHECK(gg_pack_frag(E, H, F, pk.p, gg_packed_bytes(E, H, F), fr2.p, 1 << 20, s) == GG_ERR_INVALID_ARGUMENT);
    CHECK(gg_pack_frag(E2, H2, F2, pk2.p, gg_packed_bytes(E2, H2, F2), pk2.p + 16, gg_frag_bytes(E2, H2, F2), s) ==
          GG_ERR_ALIASING);
}

static void test_noalloc() {
    const int64_t E = 2, H = 256, F = 128, M = 33;
    Buf dy(M * H * 2), h1(M * 2 * F * 2), off((E + 1) * 8), pk(gg_packed_bytes(E, H, F)), dx(M * H * 2);
    g_launches.clear();
    CHECK(gg_dgrad_noalloc(dy.p, h1.p, off.as<int64_t>(), M, pk.p, E, H, F, dx.p, fake_stream(1)) == GG_OK);
    CHECK(g_launches.size() == 2);
    if (g_launches.size() == 2) {
        // dH1 in the device's scratch array, read back by the dX GEMM
        uint16_t* scratch = g_launches[0].p.out0;
        CHECK(scratch != nullptr && g_launches[1].p.act == scratch && g_launches[1].p.out0 == dx.as<uint16_t>());
        CHECK((reinterpret_cast<uintptr_t>(scratch) & 15u) == 0);
        // the same array on the next call on that device, another on another device
        g_launches.clear();
        CHECK(gg_dgrad_noalloc(dy.p, h1.p, off.as<int64_t>(), M - 5, pk.p, E, H, F, dx.p, fake_stream(1)) == GG_OK);
        CHECK(g_launches.size() == 2 && g_launches[0].p.out0 == scratch);
        g_launches.clear();
        CHECK(gg_dgrad_noalloc(dy.p, h1.p, off.as<int64_t>(), M, pk.p, E, H, F, dx.p, fake_stream(2)) == GG_OK);
        CHECK(g_launches.size() == 2 && g_launches[0].p.out0 != scratch);
    }
    // beyond the scratch size: refused before anything else; M == 0: nothing
    g_launches.clear();
    const int64_t big_m = (int64_t(GG_NOALLOC_SCRATCH_BYTES) / (4 * F)) + 1;
    CHECK(gg_dgrad_noalloc(dy.p, h1.p, off.as<int64_t>(), big_m, pk.p, E, H, F, dx.p, fake_stream(1)) ==
          GG_ERR_WORKSPACE_TOO_SMALL);
    CHECK(gg_dgrad_noalloc(dy.p, h1.p, off.as<int64_t>(), big_m - 1, pk.p, E, H, F, dx.p + 2, fake_stream(1)) ==
          GG_ERR_MISALIGNED);
    CHECK(gg_dgrad_noalloc(nullptr, nullptr, nullptr, 0, nullptr, E, H, F, nullptr, fake_stream(1)) == GG_OK);
    CHECK(gg_dgrad_noalloc(dy.p, nullptr, off.as<int64_t>(), M, pk.p, E, H, F, dx.p, fake_stream(1)) ==
          GG_ERR_INVALID_ARGUMENT);
    CHECK(gg_dgrad_noalloc(dy.p, h1.p, off.as<int64_t>(), M, pk.p, E, H, F, dy.p + 64, fake_stream(1)) ==
          GG_ERR_ALIASING);
    CHECK(g_launches.empty());
}

static void test_scale_rows() {
    const int64_t M = 12, H = 40;
    Buf x(M * H * 2), g(M * H * 2), out(M * H * 2), dx(M * H * 2), pr(M * 4), dp(M * 4);
    hipStream_t s = fake_stream(0);
    g_launches.clear();
    // one launch each, in place allowed, dprobs optional
    CHECK(gg_scale_rows(x.p, pr.as<float>(), M, H, out.p, s) == GG_OK);
    CHECK(gg_scale_rows(x.p, pr.as<float>(), M, H, x.p, s) == GG_OK);
    CHECK(gg_scale_rows_backward(g.p, x.p, pr.as<float>(), M, H, dx.p, dp.as<float>(), s) == GG_OK);
    CHECK(gg_scale_rows_backward(g.p, x.p, pr.as<float>(), M, H, g.p, nullptr, s) == GG_OK);
    CHECK(g_launches.size() == 4);
    if (g_launches.size() == 4) {
        CHECK(!std::strcmp(g_launches[0].kind, "scale_rows") && g_launches[0].a == M && g_launches[0].b == H);
        CHECK(!std::strcmp(g_launches[2].kind, "scale_rows_bwd") && g_launches[2].c == 1 && g_launches[3].c == 0);
    }
    // argument errors launch nothing; M == 0 needs no pointers
    g_launches.clear();
    CHECK(gg_scale_rows(nullptr, nullptr, 0, H, nullptr, s) == GG_OK);
    CHECK(gg_scale_rows(x.p, pr.as<float>(), M, 36, out.p, s) == GG_ERR_INVALID_ARGUMENT);
    CHECK(gg_scale_rows(x.p, pr.as<float>(), M, H, x.p + 16, s) == GG_ERR_ALIASING);
    CHECK(gg_scale_rows(x.p, reinterpret_cast<float*>(pr.p + 2), M, H, out.p, s) == GG_ERR_MISALIGNED);
    CHECK(gg_scale_rows_backward(g.p, x.p, pr.as<float>(), M, H, x.p, nullptr, s) == GG_ERR_ALIASING);
    CHECK(gg_scale_rows_backward(g.p, x.p, pr.as<float>(), M, H, dx.p, reinterpret_cast<float*>(dx.p + 64), s) ==
          GG_ERR_ALIASING);
    CHECK(g_launches.empty());
    // the device check applies as to every call
    fake_set_arch(3, "gfx942");
    CHECK(gg_scale_rows(x.p, pr.as<float>(), M, H, out.p, fake_stream(3)) == GG_ERR_UNSUPPORTED_DEVICE);
    CHECK(g_launches.empty());
}

int main() {
    test_sizes();
    test_argument_checks();
    test_forward_launches();
    test_dgrad_launches();
    test_devices();
    test_debug_validate();
    test_pack();
    test_noalloc();
    test_scale_rows();
    std::printf("api_driver: %d of %d checks failed\n", g_failed, g_checked);
    return g_failed == 0 ? 0 : 1;
}
