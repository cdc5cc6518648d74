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
// Weighted and QuickGeGLU variants (paged-stash pull request, "What does this
// PR do" and "Validation": the fused activation is SwiGLU or QuickGeGLU, and
// its weighted form takes the router probability of each routed row at the
// activation boundary).  The pages name these activations but print no
// formula; the reading used here is
//     act(g) = g * sigmoid(c g),  c = 1 (SwiGLU) or 1.702 (QuickGeGLU)
//     A      = p_r * act(gate) * up                 (p_r omitted: p_r = 1)
//     dA     = dY W2_e
//     dH1    = [p_r dA up act'(gate) | p_r dA act(gate)]
//     dp_r   = sum_j dA[r, j] act(gate[r, j]) up[r, j]
// with act'(g) = s (1 + c g (1 - s)), s = sigmoid(c g).  dp is an fp32 sum
// over j in increasing order and is not rounded to bf16.
//
// Router probability on the FC1 input (paged-stash pull request, "What does
// this PR do": the optional multiply by the probability before FC1, the
// other of the two places a router probability enters).  No formula is
// printed; the reading used here scales the routed row before FC1, after
// which the expert MLP runs with the plain activation:
//     x'_r  = p_r x_r
// and, given g = dL/dx' (the input gradient of the MLP at x'),
//     dx_r  = p_r g_r
//     dp_r  = sum_h g[r, h] x[r, h]        (increasing h, not rounded)
// In the float instantiation x' and dx are the fp32 products rounded once
// to bf16, as every other stage.
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

// Gated activations: 0 = SwiGLU, 1 = QuickGeGLU.
enum { ACT_SWIGLU = 0, ACT_QGEGLU = 1 };

// Slope c inside the sigmoid of the gate activation.
template <typename T> T act_slope(int act) { return act == ACT_QGEGLU ? T(1.702) : T(1); }

// act(g) = g * sigmoid(c g), written as g / (1 + exp(-c g)).  For SwiGLU c g is
// g itself (c = 1 is exact).
template <typename T> T gate_act(int act, T g) { return g / (T(1) + std::exp(-(act_slope<T>(act) * g))); }

// Activation for one routed row r: A[r, j] = p_r * act(gate) * up with
// gate = H1[r, j], up = H1[r, F + j] (the rounded H1 values); without probs
// the product is act(gate) * up alone.
template <typename T>
void glu_row(int64_t r, int64_t F, int act, const T* probs, const T* h1, T* a) {
    const T* h1r = h1 + r * 2 * F;
    T* ar = a + r * F;
    for (int64_t j = 0; j < F; ++j) {
        const T g = h1r[j];
        const T u = h1r[F + j];
        const T v = gate_act<T>(act, g) * u;
        ar[j] = rnd<T>(probs ? probs[r] * v : v);
    }
}

// FC1 + activation for one routed row r of expert e: H1 row and A row.
template <typename T>
void fc1_glu_row(int64_t r, int64_t H, int64_t F, int act, const T* probs, const T* x, const T* w1e,
                 T* h1, T* a) {
    const T* xr = x + r * H;
    T* h1r = h1 + r * 2 * F;
    // FC1: H1[r, j] = sum_k X[r, k] * W1_e[j, k]
    for (int64_t j = 0; j < 2 * F; ++j) {
        const T* wj = w1e + j * H;
        T acc = 0;
        for (int64_t k = 0; k < H; ++k) acc += xr[k] * wj[k];
        h1r[j] = rnd<T>(acc);
    }
    glu_row<T>(r, F, act, probs, h1, a);
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
void forward_row(int64_t r, int64_t H, int64_t F, int act, const T* probs, const T* x, const T* w1e,
                 const T* w2e, T* h1, T* a, T* y) {
    fc1_glu_row<T>(r, H, F, act, probs, x, w1e, h1, a);
    fc2_row<T>(r, H, F, a, w2e, y);
}

// dA and the activation derivative for one routed row r of expert e -> dH1
// row (and dp_r when dprobs is given).  acc is scratch of F elements.
template <typename T>
void dglu_row(int64_t r, int64_t H, int64_t F, int act, const T* probs, const T* dy, const T* h1,
              const T* w2e, T* dh1, T* dprobs, T* acc) {
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
    // d gate = p dA * up * s * (1 + c g (1 - s)), d up = p dA * g * s, with
    // s = sigmoid(c g), g and up the saved (rounded) H1 values and dA rounded.
    const T c = act_slope<T>(act);
    T dp = 0;
    for (int64_t j = 0; j < F; ++j) {
        const T da = rnd<T>(acc[j]);
        const T g = h1r[j];
        const T u = h1r[F + j];
        const T s = sigmoid<T>(c * g);
        const T dap = probs ? probs[r] * da : da;
        dh1r[j] = rnd<T>(dap * u * s * (T(1) + c * g * (T(1) - s)));
        dh1r[F + j] = rnd<T>(dap * g * s);
        if (dprobs) dp += da * (gate_act<T>(act, g) * u);
    }
    if (dprobs) dprobs[r] = dp;
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
void dgrad_row(int64_t r, int64_t H, int64_t F, int act, const T* probs, const T* dy, const T* h1,
               const T* w1e, const T* w2e, T* dh1, T* dx, T* dprobs, T* acc) {
    dglu_row<T>(r, H, F, act, probs, dy, h1, w2e, dh1, dprobs, acc);
    dgrad_fc1_row<T>(r, H, F, dh1, w1e, dx, acc);
}

template <typename T>
void forward_all(int64_t E, int64_t H, int64_t F, const int64_t* off, int act, const T* probs,
                 const T* x, const T* w1, const T* w2, T* h1, T* a, T* y) {
    for (int64_t e = 0; e < E; ++e) {
        const T* w1e = w1 + e * 2 * F * H;
        const T* w2e = w2 + e * H * F;
#pragma omp parallel for schedule(static)
        for (int64_t r = off[e]; r < off[e + 1]; ++r)
            forward_row<T>(r, H, F, act, probs, x, w1e, w2e, h1, a, y);
    }
}

template <typename T>
void dgrad_all(int64_t E, int64_t H, int64_t F, const int64_t* off, int act, const T* probs,
               const T* dy, const T* h1, const T* w1, const T* w2, T* dh1, T* dx, T* dprobs) {
    const int64_t n_acc = H > F ? H : F;
    for (int64_t e = 0; e < E; ++e) {
        const T* w1e = w1 + e * 2 * F * H;
        const T* w2e = w2 + e * H * F;
#pragma omp parallel
        {
            std::vector<T> acc(n_acc);
#pragma omp for schedule(static)
            for (int64_t r = off[e]; r < off[e + 1]; ++r)
                dgrad_row<T>(r, H, F, act, probs, dy, h1, w1e, w2e, dh1, dx, dprobs, acc.data());
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

// x'_r = p_r x_r for every row r < M (x, out [M][H], probs [M]).
template <typename T>
void scale_rows_all(int64_t M, int64_t H, const T* probs, const T* x, T* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < M; ++r)
        for (int64_t h = 0; h < H; ++h) out[r * H + h] = rnd<T>(probs[r] * x[r * H + h]);
}

// Its input gradient: dx_r = p_r g_r and dp_r = sum_h g[r, h] x[r, h].
template <typename T>
void scale_rows_bwd_all(int64_t M, int64_t H, const T* probs, const T* g, const T* x, T* dx, T* dprobs) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < M; ++r) {
        T s = 0;
        for (int64_t h = 0; h < H; ++h) {
            dx[r * H + h] = rnd<T>(probs[r] * g[r * H + h]);
            s += g[r * H + h] * x[r * H + h];
        }
        if (dprobs) dprobs[r] = s;
    }
}

}  // namespace

extern "C" {

// SwiGLU alone, from a given H1 [M][2F] -> a [M][F], rows [offsets[0], offsets[E]).
void oracle_swiglu_f32(int64_t E, int64_t F, const int64_t* offsets, const float* h1, float* a) {
#pragma omp parallel for schedule(static)
    for (int64_t r = offsets[0]; r < offsets[E]; ++r) glu_row<float>(r, F, ACT_SWIGLU, nullptr, h1, a);
}

// Weighted / QuickGeGLU activation alone, from a given H1: act 0 = SwiGLU,
// 1 = QuickGeGLU; probs [M] fp32 or null.
void oracle_glu_f32(int64_t E, int64_t F, const int64_t* offsets, int act, const float* probs,
                    const float* h1, float* a) {
#pragma omp parallel for schedule(static)
    for (int64_t r = offsets[0]; r < offsets[E]; ++r) glu_row<float>(r, F, act, probs, h1, a);
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
    forward_all<float>(E, H, F, offsets, ACT_SWIGLU, nullptr, x, w1, w2, h1, a, y);
}

// Input gradient, fp32 accumulation with bf16 rounding points.
// dy [M][H], h1 [M][2F] (saved by the forward) -> dh1 [M][2F], dx [M][H].
void oracle_dgrad_f32(int64_t E, int64_t H, int64_t F, const int64_t* offsets,
                      const float* dy, const float* h1, const float* w1, const float* w2,
                      float* dh1, float* dx) {
    dgrad_all<float>(E, H, F, offsets, ACT_SWIGLU, nullptr, dy, h1, w1, w2, dh1, dx, nullptr);
}

// The same two passes in fp64 without rounding (finite-difference tests).
void oracle_forward_f64(int64_t E, int64_t H, int64_t F, const int64_t* offsets,
                        const double* x, const double* w1, const double* w2,
                        double* h1, double* a, double* y) {
    forward_all<double>(E, H, F, offsets, ACT_SWIGLU, nullptr, x, w1, w2, h1, a, y);
}

void oracle_dgrad_f64(int64_t E, int64_t H, int64_t F, const int64_t* offsets,
                      const double* dy, const double* h1, const double* w1, const double* w2,
                      double* dh1, double* dx) {
    dgrad_all<double>(E, H, F, offsets, ACT_SWIGLU, nullptr, dy, h1, w1, w2, dh1, dx, nullptr);
}

// Forward and input gradient with the activation chosen by act (0 SwiGLU,
// 1 QuickGeGLU) and optional per-row probabilities probs [M] (null: none).
// dprobs [M] (may be null) receives dp_r.
void oracle_forward_glu_f32(int64_t E, int64_t H, int64_t F, const int64_t* offsets, int act,
                            const float* probs, const float* x, const float* w1, const float* w2,
                            float* h1, float* a, float* y) {
    forward_all<float>(E, H, F, offsets, act, probs, x, w1, w2, h1, a, y);
}

void oracle_dgrad_glu_f32(int64_t E, int64_t H, int64_t F, const int64_t* offsets, int act,
                          const float* probs, const float* dy, const float* h1, const float* w1,
                          const float* w2, float* dh1, float* dx, float* dprobs) {
    dgrad_all<float>(E, H, F, offsets, act, probs, dy, h1, w1, w2, dh1, dx, dprobs);
}

void oracle_forward_glu_f64(int64_t E, int64_t H, int64_t F, const int64_t* offsets, int act,
                            const double* probs, const double* x, const double* w1, const double* w2,
                            double* h1, double* a, double* y) {
    forward_all<double>(E, H, F, offsets, act, probs, x, w1, w2, h1, a, y);
}

void oracle_dgrad_glu_f64(int64_t E, int64_t H, int64_t F, const int64_t* offsets, int act,
                          const double* probs, const double* dy, const double* h1, const double* w1,
                          const double* w2, double* dh1, double* dx, double* dprobs) {
    dgrad_all<double>(E, H, F, offsets, act, probs, dy, h1, w1, w2, dh1, dx, dprobs);
}

// Router probability on the FC1 input: x [M][H] -> out [M][H].
void oracle_scale_rows_f32(int64_t M, int64_t H, const float* probs, const float* x, float* out) {
    scale_rows_all<float>(M, H, probs, x, out);
}

// Its input gradient: g [M][H] (gradient at the scaled input), x [M][H]
// (the unscaled input) -> dx [M][H], dprobs [M] (may be null).
void oracle_scale_rows_bwd_f32(int64_t M, int64_t H, const float* probs, const float* g, const float* x,
                               float* dx, float* dprobs) {
    scale_rows_bwd_all<float>(M, H, probs, g, x, dx, dprobs);
}

void oracle_scale_rows_f64(int64_t M, int64_t H, const double* probs, const double* x, double* out) {
    scale_rows_all<double>(M, H, probs, x, out);
}

void oracle_scale_rows_bwd_f64(int64_t M, int64_t H, const double* probs, const double* g, const double* x,
                               double* dx, double* dprobs) {
    scale_rows_bwd_all<double>(M, H, probs, g, x, dx, dprobs);
}

}  // extern "C"
