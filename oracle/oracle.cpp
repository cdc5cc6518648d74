// CPU oracle for the frozen MoE expert grouped GEMM.  TEST INFRASTRUCTURE
// ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg call
// it; the product path never does.  It shares no code with the HIP library.
//
// What it computes (Megatron-LM pull request "perf(moe): add frozen grouped
// GEMM for adapter training", sections "Why this change" and "Why existing
// behavior remains safe"): for every local expert e, over that expert's
// contiguous block of routed rows, the bias-free gated expert MLP
//     H1 = X W1_e^T            (FC1, 2F outputs: gate | up, not interleaved)
//     A  = silu(gate) * up     (SwiGLU; TE device-metadata pull request,
//                               "What does this PR do": fused SwiGLU with GLU
//                               interleaving disabled)
//     Y  = A W2_e^T            (FC2)
// and, the expert weights being frozen, only the input gradient
//     dA  = dY W2_e
//     dH1 = [dA * up * silu'(gate) | dA * silu(gate)]
//     dX  = dH1 W1_e
// (no weight gradient).  The grouped kernel reaches exactly this per-expert
// result; it only removes the one-GEMM-per-expert launches ("Why this
// change"), so the oracle is that definition written out, one expert and one
// row at a time.
//
// Precision.  Two instantiations of the same code:
//   float  : inputs are bf16 values held in fp32, every sum accumulates in
//            fp32 in increasing index order, and H1, A, Y, dA, dH1, dX are
//            each rounded once to bf16 (round to nearest even).  SwiGLU and
//            its derivative read the bf16-rounded H1 and dA.  This is the
//            parity reference.
//   double : same loops in fp64 with no rounding; used by the tests for the
//            finite-difference check of the gradient.
// Products of two bf16 values are exact in fp32, so fused or unfused
// multiply-add give the same sums.
//
// Rows outside [offsets[0], offsets[E]) and rows of experts with no tokens
// are never written.  Offsets are read as given (the caller passes
// non-decreasing offsets within [0, M]).

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

// Round an fp32 value to the nearest bf16 value, ties to even; NaN becomes
// the canonical quiet NaN.  The result is returned widened back to fp32.
float round_to_bf16(float f) {
    uint32_t b;
    std::memcpy(&b, &f, 4);
    if ((b & 0x7fffffffu) > 0x7f800000u) {
        b = 0x7fc00000u;
    } else {
        const uint32_t lsb = (b >> 16) & 1u;
        b += 0x7fffu + lsb;
        b &= 0xffff0000u;
    }
    float r;
    std::memcpy(&r, &b, 4);
    return r;
}

template <typename T> T rnd(T v);
template <> float rnd<float>(float v) { return round_to_bf16(v); }
template <> double rnd<double>(double v) { return v; }

template <typename T> T sigmoid(T g) { return T(1) / (T(1) + std::exp(-g)); }
template <typename T> T silu(T g) { return g / (T(1) + std::exp(-g)); }

// SwiGLU for one routed row r: A[r, j] = silu(gate) * up with gate = H1[r, j],
// up = H1[r, F + j] (the rounded H1 values).
template <typename T>
void swiglu_row(int64_t r, int64_t F, const T* h1, T* a) {
    const T* h1r = h1 + r * 2 * F;
    T* ar = a + r * F;
    for (int64_t j = 0; j < F; ++j) {
        const T g = h1r[j];
        const T u = h1r[F + j];
        ar[j] = rnd<T>(silu<T>(g) * u);
    }
}

// FC1 + SwiGLU for one routed row r of expert e: H1 row and A row.
template <typename T>
void fc1_swiglu_row(int64_t r, int64_t H, int64_t F, const T* x, const T* w1e, T* h1, T* a) {
    const T* xr = x + r * H;
    T* h1r = h1 + r * 2 * F;
    // FC1: H1[r, j] = sum_k X[r, k] * W1_e[j, k]
    for (int64_t j = 0; j < 2 * F; ++j) {
        const T* wj = w1e + j * H;
        T acc = 0;
        for (int64_t k = 0; k < H; ++k) acc += xr[k] * wj[k];
        h1r[j] = rnd<T>(acc);
    }
    swiglu_row<T>(r, F, h1, a);
}

// FC2 for one routed row r of expert e: Y[r, n] = sum_j A[r, j] * W2_e[n, j].
template <typename T>
void fc2_row(int64_t r, int64_t H, int64_t F, const T* a, const T* w2e, T* y) {
    const T* ar = a + r * F;
    T* yr = y + r * H;
    for (int64_t n = 0; n < H; ++n) {
        const T* wn = w2e + n * F;
        T acc = 0;
        for (int64_t j = 0; j < F; ++j) acc += ar[j] * wn[j];
        yr[n] = rnd<T>(acc);
    }
}

// Forward for one routed row r of expert e.
template <typename T>
void forward_row(int64_t r, int64_t H, int64_t F, const T* x, const T* w1e, const T* w2e,
                 T* h1, T* a, T* y) {
    fc1_swiglu_row<T>(r, H, F, x, w1e, h1, a);
    fc2_row<T>(r, H, F, a, w2e, y);
}

// dA and the SwiGLU derivative for one routed row r of expert e -> dH1 row.
// acc is scratch of F elements.
template <typename T>
void dswiglu_row(int64_t r, int64_t H, int64_t F, const T* dy, const T* h1, const T* w2e, T* dh1,
                 T* acc) {
    const T* dyr = dy + r * H;
    const T* h1r = h1 + r * 2 * F;
    T* dh1r = dh1 + r * 2 * F;
    // dA[r, j] = sum_n dY[r, n] * W2_e[n, j]; each sum runs over n in
    // increasing order (the loop over j is inside only to walk W2 by rows).
    for (int64_t j = 0; j < F; ++j) acc[j] = 0;
    for (int64_t n = 0; n < H; ++n) {
        const T d = dyr[n];
        const T* wn = w2e + n * F;
        for (int64_t j = 0; j < F; ++j) acc[j] += d * wn[j];
    }
    // dSwiGLU: d gate = dA * up * s * (1 + g (1 - s)), d up = dA * g * s,
    // with s = sigmoid(g), g and up the saved (rounded) H1 values.
    for (int64_t j = 0; j < F; ++j) {
        const T da = rnd<T>(acc[j]);
        const T g = h1r[j];
        const T u = h1r[F + j];
        const T s = sigmoid<T>(g);
        dh1r[j] = rnd<T>(da * u * s * (T(1) + g * (T(1) - s)));
        dh1r[F + j] = rnd<T>(da * g * s);
    }
}

// dX for one routed row r of expert e: dX[r, k] = sum_j dH1[r, j] * W1_e[j, k],
// j in increasing order.  acc is scratch of H elements.
template <typename T>
void dgrad_fc1_row(int64_t r, int64_t H, int64_t F, const T* dh1, const T* w1e, T* dx, T* acc) {
    const T* dh1r = dh1 + r * 2 * F;
    for (int64_t k = 0; k < H; ++k) acc[k] = 0;
    for (int64_t j = 0; j < 2 * F; ++j) {
        const T d = dh1r[j];
        const T* wj = w1e + j * H;
        for (int64_t k = 0; k < H; ++k) acc[k] += d * wj[k];
    }
    T* dxr = dx + r * H;
    for (int64_t k = 0; k < H; ++k) dxr[k] = rnd<T>(acc[k]);
}

// Input gradient for one routed row r of expert e.  acc is scratch of
// max(F, H) elements.
template <typename T>
void dgrad_row(int64_t r, int64_t H, int64_t F, const T* dy, const T* h1, const T* w1e,
               const T* w2e, T* dh1, T* dx, T* acc) {
    dswiglu_row<T>(r, H, F, dy, h1, w2e, dh1, acc);
    dgrad_fc1_row<T>(r, H, F, dh1, w1e, dx, acc);
}

template <typename T>
void forward_all(int64_t E, int64_t H, int64_t F, const int64_t* off, const T* x,
                 const T* w1, const T* w2, T* h1, T* a, T* y) {
    for (int64_t e = 0; e < E; ++e) {
        const T* w1e = w1 + e * 2 * F * H;
        const T* w2e = w2 + e * H * F;
#pragma omp parallel for schedule(static)
        for (int64_t r = off[e]; r < off[e + 1]; ++r) forward_row<T>(r, H, F, x, w1e, w2e, h1, a, y);
    }
}

template <typename T>
void dgrad_all(int64_t E, int64_t H, int64_t F, const int64_t* off, const T* dy, const T* h1,
               const T* w1, const T* w2, T* dh1, T* dx) {
    const int64_t n_acc = H > F ? H : F;
    for (int64_t e = 0; e < E; ++e) {
        const T* w1e = w1 + e * 2 * F * H;
        const T* w2e = w2 + e * H * F;
#pragma omp parallel
        {
            std::vector<T> acc(n_acc);
#pragma omp for schedule(static)
            for (int64_t r = off[e]; r < off[e + 1]; ++r)
                dgrad_row<T>(r, H, F, dy, h1, w1e, w2e, dh1, dx, acc.data());
        }
    }
}

template <typename T>
void fc2_all(int64_t E, int64_t H, int64_t F, const int64_t* off, const T* a, const T* w2, T* y) {
    for (int64_t e = 0; e < E; ++e) {
        const T* w2e = w2 + e * H * F;
#pragma omp parallel for schedule(static)
        for (int64_t r = off[e]; r < off[e + 1]; ++r) fc2_row<T>(r, H, F, a, w2e, y);
    }
}

template <typename T>
void dgrad_fc1_all(int64_t E, int64_t H, int64_t F, const int64_t* off, const T* dh1, const T* w1,
                   T* dx) {
    for (int64_t e = 0; e < E; ++e) {
        const T* w1e = w1 + e * 2 * F * H;
#pragma omp parallel
        {
            std::vector<T> acc(H);
#pragma omp for schedule(static)
            for (int64_t r = off[e]; r < off[e + 1]; ++r) dgrad_fc1_row<T>(r, H, F, dh1, w1e, dx, acc.data());
        }
    }
}

}  // namespace

extern "C" {

// SwiGLU alone, from a given H1 [M][2F] -> a [M][F], rows [offsets[0], offsets[E]).
void oracle_swiglu_f32(int64_t E, int64_t F, const int64_t* offsets, const float* h1, float* a) {
#pragma omp parallel for schedule(static)
    for (int64_t r = offsets[0]; r < offsets[E]; ++r) swiglu_row<float>(r, F, h1, a);
}

// FC2 alone (the second step of the forward), from a given A [M][F] -> y [M][H].
void oracle_fc2_f32(int64_t E, int64_t H, int64_t F, const int64_t* offsets, const float* a,
                    const float* w2, float* y) {
    fc2_all<float>(E, H, F, offsets, a, w2, y);
}

// The last step of the input gradient alone, from a given dH1 [M][2F] -> dx [M][H].
void oracle_dgrad_fc1_f32(int64_t E, int64_t H, int64_t F, const int64_t* offsets,
                          const float* dh1, const float* w1, float* dx) {
    dgrad_fc1_all<float>(E, H, F, offsets, dh1, w1, dx);
}


// bf16 rounding of n fp32 values (exposed so the tests can pin it).
void oracle_round_bf16(const float* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = round_to_bf16(in[i]);
}

// Forward, fp32 accumulation with bf16 rounding points.  All arrays hold
// bf16 values widened to fp32.  x [M][H]; w1 [E][2F][H]; w2 [E][H][F];
// outputs h1 [M][2F], a [M][F], y [M][H].
void oracle_forward_f32(int64_t E, int64_t H, int64_t F, const int64_t* offsets,
                        const float* x, const float* w1, const float* w2,
                        float* h1, float* a, float* y) {
    forward_all<float>(E, H, F, offsets, x, w1, w2, h1, a, y);
}

// Input gradient, fp32 accumulation with bf16 rounding points.
// dy [M][H], h1 [M][2F] (saved by the forward) -> dh1 [M][2F], dx [M][H].
void oracle_dgrad_f32(int64_t E, int64_t H, int64_t F, const int64_t* offsets,
                      const float* dy, const float* h1, const float* w1, const float* w2,
                      float* dh1, float* dx) {
    dgrad_all<float>(E, H, F, offsets, dy, h1, w1, w2, dh1, dx);
}

// The same two passes in fp64 without rounding (finite-difference tests).
void oracle_forward_f64(int64_t E, int64_t H, int64_t F, const int64_t* offsets,
                        const double* x, const double* w1, const double* w2,
                        double* h1, double* a, double* y) {
    forward_all<double>(E, H, F, offsets, x, w1, w2, h1, a, y);
}

void oracle_dgrad_f64(int64_t E, int64_t H, int64_t F, const int64_t* offsets,
                      const double* dy, const double* h1, const double* w1, const double* w2,
                      double* dh1, double* dx) {
    dgrad_all<double>(E, H, F, offsets, dy, h1, w1, w2, dh1, dx);
}

}  // extern "C"
