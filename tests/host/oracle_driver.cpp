// Drives every exported function of oracle/oracle.cpp on small exact-size
// buffers (a read or write past any of them is caught by AddressSanitizer;
// undefined arithmetic by UndefinedBehaviorSanitizer): empty experts first,
// in the middle and last, rows before offsets[0] and after offsets[E] that
// must stay untouched, K lengths that are not multiples of anything, and
// the rounding routine on special values.  Built and run by
// tests/test_host_sanitized.py.  Exit status 0 when every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

extern "C" {
void oracle_swiglu_f32(int64_t, int64_t, const int64_t*, const float*, float*);
void oracle_glu_f32(int64_t, int64_t, const int64_t*, int, const float*, const float*, float*);
void oracle_fc2_f32(int64_t, int64_t, int64_t, const int64_t*, const float*, const float*, float*);
void oracle_dgrad_fc1_f32(int64_t, int64_t, int64_t, const int64_t*, const float*, const float*, float*);
void oracle_round_bf16(const float*, float*, int64_t);
void oracle_forward_f32(int64_t, int64_t, int64_t, const int64_t*, const float*, const float*, const float*,
                        float*, float*, float*);
void oracle_dgrad_f32(int64_t, int64_t, int64_t, const int64_t*, const float*, const float*, const float*,
                      const float*, float*, float*);
void oracle_forward_f64(int64_t, int64_t, int64_t, const int64_t*, const double*, const double*, const double*,
                        double*, double*, double*);
void oracle_dgrad_f64(int64_t, int64_t, int64_t, const int64_t*, const double*, const double*, const double*,
                      const double*, double*, double*);
void oracle_forward_glu_f32(int64_t, int64_t, int64_t, const int64_t*, int, const float*, const float*,
                            const float*, const float*, float*, float*, float*);
void oracle_dgrad_glu_f32(int64_t, int64_t, int64_t, const int64_t*, int, const float*, const float*,
                          const float*, const float*, const float*, float*, float*, float*);
void oracle_forward_glu_f64(int64_t, int64_t, int64_t, const int64_t*, int, const double*, const double*,
                            const double*, const double*, double*, double*, double*);
void oracle_dgrad_glu_f64(int64_t, int64_t, int64_t, const int64_t*, int, const double*, const double*,
                          const double*, const double*, const double*, double*, double*, double*);
}

static int g_failed = 0, g_checked = 0;
#define CHECK(cond)                                                                               \
    do {                                                                                          \
        ++g_checked;                                                                              \
        if (!(cond)) {                                                                            \
            ++g_failed;                                                                           \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond);          \
        }                                                                                         \
    } while (0)

// bf16 values (low 16 mantissa bits clear) from a fixed-seed generator.
static float bf16_value(uint32_t& s, float scale) {
    s = s * 1664525u + 1013904223u;
    const float u = (static_cast<float>(s >> 8) / 16777216.0f - 0.5f) * 2.0f * scale;
    uint32_t b;
    std::memcpy(&b, &u, 4);
    b &= 0xFFFF0000u;
    float v;
    std::memcpy(&v, &b, 4);
    return v;
}

template <typename T>
static bool rows_untouched(const std::vector<T>& v, int64_t cols, int64_t r0, int64_t r1) {
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = 0; c < cols; ++c)
            if (!std::isnan(v[r * cols + c])) return false;
    return true;
}

template <typename T>
static bool rows_finite(const std::vector<T>& v, int64_t cols, int64_t r0, int64_t r1) {
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = 0; c < cols; ++c)
            if (!std::isfinite(v[r * cols + c])) return false;
    return true;
}

template <typename T>
static void run(const char* tag) {
    const int64_t E = 5, H = 24, F = 40, M = 23;
    // experts 0, 2 and 4 empty; rows [0, 3) and [20, 23) outside the offsets
    const int64_t off[E + 1] = {3, 3, 11, 11, 20, 20};
    uint32_t seed = 12345;
    std::vector<T> x(M * H), dy(M * H), w1(E * 2 * F * H), w2(E * H * F), probs(M);
    for (auto& v : x) v = bf16_value(seed, 2.0f);
    for (auto& v : dy) v = bf16_value(seed, 2.0f);
    for (auto& v : w1) v = bf16_value(seed, 0.1f);
    for (auto& v : w2) v = bf16_value(seed, 0.1f);
    for (auto& v : probs) v = std::fabs(bf16_value(seed, 1.0f)) + T(0.01);
    const T nan = std::nan("");
    for (int act = 0; act < 2; ++act) {
        std::vector<T> h1(M * 2 * F, nan), a(M * F, nan), y(M * H, nan), dh1(M * 2 * F, nan), dx(M * H, nan),
            dp(M, nan);
        if constexpr (sizeof(T) == 4) {
            oracle_forward_glu_f32(E, H, F, off, act, probs.data(), x.data(), w1.data(), w2.data(), h1.data(),
                                   a.data(), y.data());
            oracle_dgrad_glu_f32(E, H, F, off, act, probs.data(), dy.data(), h1.data(), w1.data(), w2.data(),
                                 dh1.data(), dx.data(), dp.data());
        } else {
            oracle_forward_glu_f64(E, H, F, off, act, probs.data(), x.data(), w1.data(), w2.data(), h1.data(),
                                   a.data(), y.data());
            oracle_dgrad_glu_f64(E, H, F, off, act, probs.data(), dy.data(), h1.data(), w1.data(), w2.data(),
                                 dh1.data(), dx.data(), dp.data());
        }
        CHECK(rows_untouched(h1, 2 * F, 0, 3) && rows_untouched(h1, 2 * F, 20, M));
        CHECK(rows_untouched(y, H, 0, 3) && rows_untouched(dx, H, 20, M) && rows_untouched(dp, 1, 0, 3));
        CHECK(rows_finite(h1, 2 * F, 3, 20) && rows_finite(a, F, 3, 20) && rows_finite(y, H, 3, 20));
        CHECK(rows_finite(dh1, 2 * F, 3, 20) && rows_finite(dx, H, 3, 20) && rows_finite(dp, 1, 3, 20));
    }
    // the plain passes, and the single stages of the fp32 instantiation
    std::vector<T> h1(M * 2 * F, nan), a(M * F, nan), y(M * H, nan), dh1(M * 2 * F, nan), dx(M * H, nan);
    if constexpr (sizeof(T) == 4) {
        oracle_forward_f32(E, H, F, off, x.data(), w1.data(), w2.data(), h1.data(), a.data(), y.data());
        oracle_dgrad_f32(E, H, F, off, dy.data(), h1.data(), w1.data(), w2.data(), dh1.data(), dx.data());
        std::vector<T> a2(M * F, nan), a3(M * F, nan), y2(M * H, nan), dx2(M * H, nan);
        oracle_swiglu_f32(E, F, off, h1.data(), a2.data());
        oracle_glu_f32(E, F, off, 0, nullptr, h1.data(), a3.data());
        oracle_fc2_f32(E, H, F, off, a.data(), w2.data(), y2.data());
        oracle_dgrad_fc1_f32(E, H, F, off, dh1.data(), w1.data(), dx2.data());
        // the stages compose to the whole passes, bit for bit
        CHECK(std::memcmp(a2.data() + 3 * F, a.data() + 3 * F, 17 * F * sizeof(T)) == 0);
        CHECK(std::memcmp(a3.data() + 3 * F, a.data() + 3 * F, 17 * F * sizeof(T)) == 0);
        CHECK(std::memcmp(y2.data() + 3 * H, y.data() + 3 * H, 17 * H * sizeof(T)) == 0);
        CHECK(std::memcmp(dx2.data() + 3 * H, dx.data() + 3 * H, 17 * H * sizeof(T)) == 0);
    } else {
        oracle_forward_f64(E, H, F, off, x.data(), w1.data(), w2.data(), h1.data(), a.data(), y.data());
        oracle_dgrad_f64(E, H, F, off, dy.data(), h1.data(), w1.data(), w2.data(), dh1.data(), dx.data());
    }
    CHECK(rows_untouched(a, F, 0, 3) && rows_finite(dx, H, 3, 20) && rows_untouched(dx, H, 20, M));
    std::printf("oracle_driver: %s passes done\n", tag);
}

int main() {
    run<float>("fp32");
    run<double>("fp64");
    // rounding: special values, ties, subnormals, overflow to infinity
    const float in[] = {0.0f, -0.0f, 1.0f, 1.00390625f /* tie, even down */, 1.01171875f /* tie, even up */,
                        1e-40f, -1e-45f, 3.4e38f, INFINITY, -INFINITY, NAN};
    const int n = sizeof(in) / sizeof(in[0]);
    std::vector<float> out(n);
    oracle_round_bf16(in, out.data(), n);
    CHECK(out[2] == 1.0f && out[3] == 1.0f && out[4] == 1.015625f);
    CHECK(std::isinf(out[7]) && std::isinf(out[8]) && std::isinf(out[9]) && std::isnan(out[10]));
    CHECK(std::signbit(out[1]) && out[0] == 0.0f);
    std::printf("oracle_driver: %d of %d checks failed\n", g_failed, g_checked);
    return g_failed == 0 ? 0 : 1;
}
