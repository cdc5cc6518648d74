/* gg.h -- C ABI of the MI355X (gfx950) grouped GEMM for frozen MoE experts.
 *
 * The library runs, for every local expert e over that expert's contiguous
 * block of routed token rows, the bias-free gated expert MLP and its input
 * gradient:
 *
 *   forward   H1 = X W1_e^T          [rows, 2F]  gate = H1[:, :F], up = H1[:, F:]
 *             A  = silu(gate) * up   [rows, F]
 *             Y  = A W2_e^T          [rows, H]
 *   dgrad     dA  = dY W2_e                                 [rows, F]
 *             dH1 = [dA * up * silu'(gate) | dA * silu(gate)] [rows, 2F]
 *             dX  = dH1 W1_e                                [rows, H]
 *
 * with all experts covered by one launch per GEMM, as the Megatron-LM pull
 * request "perf(moe): add frozen grouped GEMM for adapter training" does in
 * place of one small GEMM per expert (section "Why this change").  Weights
 * are frozen, grouped, bias-free BF16 (section "Why existing behavior remains
 * safe"), so there is no weight gradient.  Per-expert row counts stay on the
 * device and are never read by the host (TE device-metadata grouped GEMM
 * pull request, section "Summary").  The gated activation is SwiGLU with the
 * gate and up halves as two contiguous blocks, not interleaved (paged-stash
 * pull request, section "What does this PR do").
 *
 * Conventions shared by every call
 *  - Tensors are DEVICE pointers to bf16 bit patterns, row-major, 16-byte
 *    aligned.  `offsets` is a DEVICE pointer to E+1 int64 values.  Every
 *    buffer of a call lies on the stream's device (the current device for
 *    the null stream), where the call's kernels run; the library does not
 *    look up which device a pointer belongs to.
 *  - Rows are sorted by expert: expert e owns rows [offsets[e], offsets[e+1]).
 *    offsets must be non-decreasing with 0 <= offsets[0] and offsets[E] <= M.
 *    An expert with offsets[e] == offsets[e+1] has no tokens: nothing is read
 *    from its weights and nothing is written for it.  The kernels clamp each
 *    offset into [0, M] and treat a decreasing pair as empty, so bad offsets
 *    cannot cause an out-of-bounds access (results are then undefined).
 *  - Outputs are written only at rows [offsets[0], offsets[E]); other rows
 *    keep their contents.
 *  - Packed weights: one buffer, expert-major, per expert e
 *      W1_e [2F][H] at element offset e*3*F*H   (rows 0..F-1 gate, F..2F-1 up)
 *      W2_e [H][F]  at element offset e*3*F*H + 2*F*H
 *    (runtime packing of frozen expert weights into one contiguous buffer,
 *    "Artifacts" and "Why existing behavior remains safe" of the first page).
 *  - Ownership: the caller owns every buffer.  The library allocates nothing
 *    on these calls, keeps no pointer after returning, and never synchronises
 *    the host: every call is asynchronous on `stream`.
 *  - Errors: every call returns a gg_status and never aborts.  Argument
 *    checks run before any HIP call.  M == 0 returns GG_OK without a launch.
 *    A device that is not gfx950 gives GG_ERR_UNSUPPORTED_DEVICE (other
 *    GPU/library pairs fail explicitly, TE device-metadata pull request,
 *    "Summary").  Launch failures give GG_ERR_HIP.
 *  - Limits: 1 <= E <= GG_MAX_EXPERTS; H and F positive multiples of 8;
 *    H < 2^22 and 2F < 2^22; one expert's W1 below 2 GiB (4*F*H < 2^31
 *    bytes); M < 2^31.
 */
#ifndef GG_H_
#define GG_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GG_MAX_EXPERTS 1024

typedef enum {
    GG_OK = 0,
    GG_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, E/H/F/M out of range */
    GG_ERR_MISALIGNED = 2,         /* a tensor pointer is not 16-byte aligned */
    GG_ERR_UNSUPPORTED_DEVICE = 3, /* the stream's device (the current device for the null stream) is not gfx950 */
    GG_ERR_WORKSPACE_TOO_SMALL = 4,/* packed_bytes or workspace_bytes too small */
    GG_ERR_ALIASING = 5,           /* an output overlaps an input or another output */
    GG_ERR_HIP = 6                 /* a HIP runtime call failed */
} gg_status;

/* Human-readable name of a status code (static string). */
const char* gg_status_string(int status);

/* Bytes of the packed weight buffer: 6*E*H*F.  Expert-major blocks of 3*F*H
 * bf16 elements: W1_e [2F][H] at element offset e*3*F*H, then W2_e [H][F]
 * at e*3*F*H + 2*F*H, both row-major.  One expert block (or any contiguous
 * range of them) is itself a packed buffer with E = 1 (or the range's E).
 * Returns 0 when E, H or F is not positive. */
size_t gg_packed_bytes(int64_t E, int64_t H, int64_t F);

/* Bytes of the gg_dgrad workspace: dH1 [M][2F] bf16 = 4*M*F. */
size_t gg_dgrad_workspace_bytes(int64_t M, int64_t F);

/* Pack E experts' frozen weights into `packed` (expert-major layout above),
 * so that every expert's parameters can become views into one contiguous
 * buffer, as the runtime packing of frozen expert weights does in the first
 * page ("Artifacts" and "Why existing behavior remains safe", which also note
 * an unchanged peak allocated memory: the buffer is exactly the weights).
 * w1, w2: HOST arrays of E DEVICE pointers; w1[e] -> [2F][H], w2[e] -> [H][F].
 * A source that already is its destination inside `packed` is skipped, so
 * re-packing after one expert's weights were replaced copies only what
 * moved (recovery after a middle expert weight is replaced, same section).
 * A source that partially overlaps `packed` gives GG_ERR_ALIASING.  Copies
 * are asynchronous device-to-device on `stream`.  packed_bytes is the size
 * of `packed` (at least gg_packed_bytes(E, H, F)). */
int gg_pack_weights(int64_t E, int64_t H, int64_t F,
                    const void* const* w1, const void* const* w2,
                    void* packed, size_t packed_bytes, hipStream_t stream);

/* ---- Opt-in fragment-ordered weight copies (this library's own layout;
 * the pages pack only the original matrices).  For shapes with H % 256 == 0
 * and F % 128 == 0, a second, caller-owned buffer can hold copies of every
 * expert's W1, W2, W1^T and W2^T in the operand order of the CDNA4 bf16
 * matrix instruction, which lets the four GEMMs load their weight operands
 * straight into registers.  The extended calls below take it as `frag`
 * (NULL: not used).  It costs 12*E*H*F more bytes (twice the weights) and
 * on MI355X saves 13-25% of the FC1, FC2 and dX time and 26-29% of dA's on
 * large workloads (H = 2048-4096).  The copies are derived from the packed
 * buffer by gg_pack_frag and do not follow later writes to it: call
 * gg_pack_frag again after re-packing. */

/* Bytes of the fragment buffer: 12*E*H*F when H % 256 == 0 and F % 128 == 0,
 * 0 for every other shape (no copies exist for it). */
size_t gg_frag_bytes(int64_t E, int64_t H, int64_t F);

/* Write the fragment-ordered copies of the E experts of `packed` into
 * `frag` (DEVICE, 16-byte aligned, frag_bytes >= gg_frag_bytes(E, H, F)).
 * Asynchronous on `stream`.  GG_ERR_INVALID_ARGUMENT for a shape without
 * copies; GG_ERR_ALIASING if the buffers overlap. */
int gg_pack_frag(int64_t E, int64_t H, int64_t F, const void* packed, size_t packed_bytes,
                 void* frag, size_t frag_bytes, hipStream_t stream);

/* Forward FC1 with the fused SwiGLU epilogue.
 * x [M][H]; packed as above; h1_out [M][2F] (the bf16 FC1 output, saved for
 * the gradient; may be NULL when no gradient follows); a_out [M][F] =
 * bf16(silu(gate) * up) computed from the bf16-rounded gate and up. */
int gg_forward_fc1_swiglu(const void* x, const int64_t* offsets, int64_t M,
                          const void* packed, int64_t E, int64_t H, int64_t F,
                          void* h1_out, void* a_out, hipStream_t stream);

/* Forward FC2: y [M][H] = A W2_e^T per expert, a [M][F]. */
int gg_forward_fc2(const void* a, const int64_t* offsets, int64_t M,
                   const void* packed, int64_t E, int64_t H, int64_t F,
                   void* y, hipStream_t stream);

/* Input gradient of the whole expert MLP (frozen weights: no weight
 * gradient; "input gradient" parity of the first page's "Artifacts").
 * dy [M][H]; h1 [M][2F] as written by gg_forward_fc1_swiglu; workspace of at
 * least gg_dgrad_workspace_bytes(M, F) bytes receives dH1 [M][2F];
 * dx [M][H] receives the input gradient.  Two launches on `stream`. */
int gg_dgrad(const void* dy, const void* h1, const int64_t* offsets, int64_t M,
             const void* packed, int64_t E, int64_t H, int64_t F,
             void* workspace, size_t workspace_bytes, void* dx, hipStream_t stream);

/* ---- Weighted SwiGLU / QuickGeGLU (paged-stash pull request, "What does
 * this PR do" and "Validation": the fused activation is SwiGLU or QuickGeGLU,
 * and its weighted form takes each routed row's router probability at the
 * activation boundary).  The pages give no formula; this library reads them as
 *   act(g) = g * sigmoid(c g),  c = 1 (GG_ACT_SWIGLU) or 1.702 (GG_ACT_QGEGLU)
 *   A      = bf16(p_r * act(gate) * up)        (probs == NULL: p_r = 1)
 *   dH1    = [p_r dA up act'(gate) | p_r dA act(gate)]
 *   dp_r   = sum_j dA[r, j] act(gate[r, j]) up[r, j]   (fp32, not rounded)
 * with gate, up the bf16 H1 values and dA = bf16(dY W2_e).  The sum of dp_r
 * is taken in a fixed order (32-column groups in increasing order, each
 * group in a fixed lane order), so dp_r, like every other output, does not
 * depend on the rest of the batch. */
typedef enum {
    GG_ACT_SWIGLU = 0,
    GG_ACT_QGEGLU = 1
} gg_activation;

/* Bytes of the gg_dgrad_glu workspace: dH1 [M][2F] bf16 (4*M*F), plus, when
 * dp is requested, 4*M*ceil(F/32) bytes of fp32 partial sums. */
size_t gg_dgrad_glu_workspace_bytes(int64_t M, int64_t F, int with_dprobs);

/* gg_forward_fc1_swiglu with the activation chosen by `activation` (a
 * gg_activation) and, when `probs` is not NULL, each routed row's activation
 * scaled by probs[r] (DEVICE fp32 [M], 4-byte aligned, read only).  `frag`
 * is NULL or the fragment buffer of the same weights (gg_pack_frag); the
 * results do not depend on it, bit for bit.  An unknown activation, or a
 * frag for a shape without copies, gives GG_ERR_INVALID_ARGUMENT.  With
 * GG_ACT_SWIGLU and probs == NULL the results are those of
 * gg_forward_fc1_swiglu, bit for bit. */
int gg_forward_fc1_glu(const void* x, const int64_t* offsets, int64_t M,
                       const void* packed, const void* frag, int64_t E, int64_t H, int64_t F,
                       int activation, const float* probs,
                       void* h1_out, void* a_out, hipStream_t stream);

/* gg_forward_fc2 with an optional fragment buffer (`frag` as in
 * gg_forward_fc1_glu); the results are those of gg_forward_fc2, bit for bit. */
int gg_forward_fc2_frag(const void* a, const int64_t* offsets, int64_t M,
                        const void* packed, const void* frag, int64_t E, int64_t H, int64_t F,
                        void* y, hipStream_t stream);

/* Input gradient of gg_forward_fc1_glu + gg_forward_fc2: as gg_dgrad, with
 * the same `activation` and `probs` as the forward.  dprobs (DEVICE fp32 [M],
 * 4-byte aligned, or NULL) receives dp_r for the routed rows; the workspace
 * must then hold gg_dgrad_glu_workspace_bytes(M, F, 1) bytes (dH1 first, then
 * the partial sums).  Two launches on `stream`, three with dprobs.  With
 * GG_ACT_SWIGLU, probs == NULL and dprobs == NULL the results are those of
 * gg_dgrad, bit for bit.  `frag` as in gg_forward_fc1_glu (used by the dX
 * GEMM, and by dA when F % 256 == 0, for every activation and with or
 * without probs; the results, dprobs included, do not depend on it). */
int gg_dgrad_glu(const void* dy, const void* h1, const int64_t* offsets, int64_t M,
                 const void* packed, const void* frag, int64_t E, int64_t H, int64_t F,
                 int activation, const float* probs,
                 void* workspace, size_t workspace_bytes, void* dx, float* dprobs,
                 hipStream_t stream);

/* Input gradient without a saved H1: recomputes FC1 from x (the forward's
 * input, [M][H]) inside the call, for a forward run with h1_out == NULL.
 * This is the trade of selective `expert_fc1_act` recompute (Megatron-LM
 * pull request "perf(moe): add frozen grouped GEMM for adapter training",
 * section "Scope deliberately omitted"; issue "feat(moe+ssm): expert-LoRA
 * GEMM stack and hybrid-recompute guard", section "What's in it"): 4*M*F
 * bytes of H1 are not kept between the forward and the backward, at the
 * price of 4*M*H*F more FLOPs here.  Three launches on `stream` (four with dprobs):
 * H1 = X W1_e^T into the workspace, then dA and the activation derivative
 * overwrite it in place with dH1, then dX.  The workspace size is
 * gg_dgrad_glu_workspace_bytes(M, F, dprobs != NULL), the same as with a
 * saved H1.  The recomputed H1 is bit-identical to the forward's, so dx and
 * dprobs equal those of gg_dgrad_glu with the saved H1, bit for bit.
 * Other arguments as gg_dgrad_glu. */
int gg_dgrad_recompute(const void* dy, const void* x, const int64_t* offsets, int64_t M,
                       const void* packed, const void* frag, int64_t E, int64_t H, int64_t F,
                       int activation, const float* probs,
                       void* workspace, size_t workspace_bytes, void* dx, float* dprobs,
                       hipStream_t stream);

/* ---- Router probability on the FC1 input.  The paged-stash pull request
 * ("[Main] Support paged stash with device-initiated GroupedLinear", "What
 * does this PR do") names two places where a routed row's probability can
 * enter the expert MLP: the activation boundary (gg_forward_fc1_glu's probs)
 * and an optional multiply before FC1, which the fused path does not run.
 * These two calls are that multiply and its input gradient, for use around
 * the plain calls (gg_forward_fc1_swiglu ... gg_dgrad on the scaled rows).
 * The pages give no formula; this library reads them as
 *   x'[r][h]  = bf16(p_r * x[r][h])            (fp32 product, nearest even)
 *   dx[r][h]  = bf16(p_r * dxs[r][h])          (dxs = dL/dx', e.g. gg_dgrad's dx)
 *   dprobs[r] = sum_h dxs[r][h] * x[r][h]      (fp32, not rounded)
 * for every row r < M (not only the routed ones; there are no offsets).
 * x, x_out, dxs, dx: DEVICE bf16 [M][H], 16-byte aligned; probs, dprobs:
 * DEVICE fp32 [M], 4-byte aligned.  H % 8 == 0, else GG_ERR_INVALID_ARGUMENT.
 * x_out may be x, and dx may be dxs (in place); any other overlap of an
 * output with an input or another output gives GG_ERR_ALIASING.  dprobs may
 * be NULL.  The sum of dprobs[r] has one fixed order (one wavefront per row:
 * lane l adds 16-byte chunks l, l + 64, ... in increasing h, then the lane
 * sums are combined pairwise, lanes 32 apart first).  One launch on
 * `stream` each; M == 0 returns GG_OK without one. */
int gg_scale_rows(const void* x, const float* probs, int64_t M, int64_t H, void* x_out, hipStream_t stream);
int gg_scale_rows_backward(const void* dxs, const void* x, const float* probs, int64_t M, int64_t H,
                           void* dx, float* dprobs, hipStream_t stream);

/* ---- For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).
 * gg_dgrad without a workspace argument: dH1 goes to a static device array
 * of the library, GG_NOALLOC_SCRATCH_BYTES bytes per GPU, allocated when the
 * library's code is loaded on that GPU and held until the process ends.  The
 * call allocates nothing and needs 4*M*F <= GG_NOALLOC_SCRATCH_BYTES
 * (GG_ERR_WORKSPACE_TOO_SMALL otherwise; M*F <= 32 Mi elements).  Every call
 * on one GPU uses that GPU's one array, so calls that overlap on one GPU
 * (concurrent streams, or host threads) race and give undefined results:
 * serialise them on one stream.  Nothing in the array needs clearing
 * between calls.  Other arguments and results as gg_dgrad, bit for bit. */
#define GG_NOALLOC_SCRATCH_BYTES (128u << 20)
int gg_dgrad_noalloc(const void* dy, const void* h1, const int64_t* offsets, int64_t M,
                     const void* packed, int64_t E, int64_t H, int64_t F,
                     void* dx, hipStream_t stream);

/* Diagnostic: round n fp32 values to bf16 on the device with the same
 * conversion the epilogues use (lets a test check the device rounding
 * against round-to-nearest-even).  in: DEVICE float[n]; out: DEVICE
 * uint16[n]; asynchronous on `stream`. */
int gg_round_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GG_H_ */
