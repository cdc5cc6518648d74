// Internal interface between the C-ABI entry points and the grouped GEMM
// kernels (not part of the public ABI; see include/gg.h for that).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define GG_KMAX_EXPERTS 1024

namespace gg {

enum Epilogue { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2 };

// One grouped GEMM over all experts: for expert e and its rows r,
//   out[r, n] = sum_k act[r, k] * Wt_e[n, k]   (Wt_e[n, k] = W_e[n*ldw + k] when the
//               weights are K-contiguous, W_e[k*ldw + n] for the transposed variant)
struct GemmParams {
    const uint16_t* act;       // token operand [M][K] (X, A, dY or dH1), row stride K
    const uint16_t* w;         // packed weights + in-expert offset of this GEMM's matrix
    const int64_t* offsets;    // device [E+1]
    int64_t w_expert_stride;   // elements between consecutive experts (3*F*H)
    int M, E, K, N;            // N = output columns (F for the SwiGLU variants)
    int ldw;                   // weight row stride in elements
    int up_off;                // SwiGLU: row index of the first "up" row of W1 (= F)
    uint16_t* out0;            // Y / dX, or A (SwiGLU), or dH1 [M][2F] (SwiGLU derivative)
    uint16_t* out1;            // SwiGLU: H1 [M][2F] or null
    const uint16_t* aux;       // SwiGLU derivative: saved H1 [M][2F]
    // Gated activation act(g) = g * sigmoid(slope * g): slope 1 is SwiGLU,
    // 1.702 QuickGeGLU.
    float slope;
    const float* probs;        // per-row weight of the activation [M], or null
    float* dp_part;            // derivative variant: partial sums of dp per row and
                               // 32-column group [M][dp_ld], or null
    int dp_ld;                 // ceil(N / 32)
    // This GEMM's matrix in the caller's fragment-ordered copy of the weights,
    // or null.  With it, the GEMM runs in the four-wave kernel (dgrad FC2: F a
    // multiple of 256).
    const uint16_t* wfrag;
    int64_t wfrag_stride;      // elements between consecutive experts in the fragment copy
    int h1_order;              // plain store over W1's fragment copy: write the columns in H1's gate | up order
};

hipError_t launch_fc1_swiglu(const GemmParams& p, int num_cu, hipStream_t s);
hipError_t launch_fc2(const GemmParams& p, int num_cu, hipStream_t s);
hipError_t launch_dgrad_fc2(const GemmParams& p, int num_cu, hipStream_t s);
hipError_t launch_dgrad_fc1(const GemmParams& p, int num_cu, hipStream_t s);
// Fragment-ordered copies of every expert's W1, W2, W1^T and W2^T (H % 256 == 0,
// F % 128 == 0), written into `frag` (FRAG_BLOCK_FH * F * H elements per expert)
// from the row-major packed buffer.
constexpr int FRAG_BLOCK_FH = 6;
constexpr int FRAG_W1 = 0, FRAG_W2 = 2, FRAG_W1T = 3, FRAG_W2T = 5;   // offsets in an expert block, units of F*H
// each matrix ends where the next begins (W1 2FH, W2 FH, W1^T 2FH, W2^T FH elements)
static_assert(FRAG_W2 - FRAG_W1 == 2 && FRAG_W1T - FRAG_W2 == 1 && FRAG_W2T - FRAG_W1T == 2 &&
                  FRAG_BLOCK_FH - FRAG_W2T == 1, "fragment block layout");
hipError_t launch_pack_frag(const uint16_t* packed, uint16_t* frag, int E, int H, int F, hipStream_t s);
hipError_t launch_round_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s);
// Router probability on the FC1 input, every row r < M: out = bf16(p_r x_r)
// (out may be x); and its input gradient dx = bf16(p_r g_r) (dx may be g),
// dprobs[r] = sum_h g x (dprobs may be null).  H % 8 == 0.
hipError_t launch_scale_rows(const uint16_t* x, const float* probs, int64_t M, int H, uint16_t* out,
                             hipStream_t s);
hipError_t launch_scale_rows_bwd(const uint16_t* g, const uint16_t* x, const float* probs, int64_t M, int H,
                                 uint16_t* dx, float* dprobs, hipStream_t s);
// Device address of the no-allocation scratch array (GG_NOALLOC_SCRATCH_BYTES)
// on `device`, looked up once per device and cached (gg_noalloc.hip).
hipError_t noalloc_scratch(int device, void** ptr);
// dprobs[r] = sum over g of part[r][g] in increasing g, for the routed rows.
hipError_t launch_dp_reduce(const int64_t* offsets, int E, int M, const float* part, int ld, float* dprobs,
                            hipStream_t s);

}  // namespace gg
