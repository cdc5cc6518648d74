// Grouped GEMM kernels for frozen MoE experts on CDNA4 (gfx950).
//
// One persistent launch covers every expert of a GEMM.  Each workgroup reads
// the int64 expert offsets from device memory, turns them into per-expert
// tile counts and an exclusive prefix sum in LDS (the per-expert sizes never
// go through the host, as in the TE device-metadata grouped GEMM pull
// request, section "Summary"), and then walks the global tile list.  Experts
// with no rows own no tiles, so their weights are never read.
//
// Two kernels.  The eight-wave kernel (grouped_gemm_kernel) runs every GEMM
// over the row-major packed weights; the four-wave kernel (tile4_kernel,
// below) runs FC1, FC2, dX and, with F a multiple of 256, the dgrad FC2 when
// the caller also passes a fragment-ordered copy of the weights.  In the
// eight-wave kernel two flavors share one launch.  Rows that fill 256-row
// tiles run as 256 x 256 output tiles; the at most 96 rows an expert leaves
// over (all rows of a small expert) run as weight-streaming items, before the
// tiles.  An item is
// those rows x 192 weight rows (six compute waves of 32 rows; two more waves
// issue every copy into a 4-stage ring), or x 96 weight rows when the items
// fit into the grid twice over, so that they spread over all workgroups.
//
// Tile core: bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulators), 8 waves
// of 128 token rows x 64 output columns.  Both operand panels stream from HBM
// straight into LDS with LDS-DMA loads (global_load_lds_dwordx4, 16 bytes per
// lane) through a 2-stage ring of 64-k stages, so the next stage is in flight
// while the matrix cores work on the current one.
//  - K-contiguous panels (tokens; forward weights) sit in LDS as [row][64 k]
//    with the eight 16-byte chunks of a row XOR-swizzled by (row >> 1) & 7;
//    fragments are read with ds_read_b128.
//  - The transposed-weight variant (dgrad) reads W as [K][N] (N contiguous):
//    the panel lands in LDS as [64 k][256 n] with 16-byte chunks swizzled by
//    (k & 3) << 2 and the MFMA operand is assembled with two
//    ds_read_b64_tr_b16 per fragment, which transpose 4x16 blocks of 16-bit
//    elements across each group of 16 lanes.
//  - Forward kernels: every wave reads the next k16 step's fragments while
//    the MFMAs of the current one issue (one barrier per stage).  Dgrad
//    kernels: the two 4-wave groups alternate ("ping-pong") between reading
//    and computing 32-k half stages.
// The weight side is the MFMA "A" operand and the token side the "B"
// operand, so each lane ends up holding one token row and four groups of
// four consecutive output columns; epilogues stage results through LDS and
// store 16-byte row segments.
//
// Variants (template parameters W_KN, EPI, EXT):
//   FC1 + SwiGLU  W_KN=false  weights W1_e [2F][H]; a tile loads matching gate
//                 rows n.. and up rows F+n.. so SwiGLU is applied in
//                 registers; writes H1 (optional) and A.
//   FC2           W_KN=false  weights W2_e [H][F]; writes Y (also the FC1
//                 recompute inside the input gradient, over W1's 2F rows).
//   dgrad FC2     W_KN=true   dA = dY W2_e (contraction over W2's rows); the
//                 epilogue applies the SwiGLU derivative with the saved H1
//                 and writes dH1.
//   dgrad FC1     W_KN=true   dX = dH1 W1_e; writes dX.
//   EXT           QuickGeGLU slope, per-row weights and dp partial sums in
//                 the FC1 and dgrad-FC2 epilogues (plain SwiGLU otherwise).
// Rounding points mirror the unfused computation: H1, A, Y, dA, dH1 and dX
// are each rounded once to bf16 (round to nearest even); SwiGLU and its
// derivative read the rounded gate/up and dA.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gg_kernels.h"

namespace gg {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

#define GG_AS3(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int BK = 64;  // K elements per pipeline stage (128-byte rows of a K-contiguous panel)
constexpr int HK = 32;  // K elements per ping-pong phase (half a stage)

__device__ __forceinline__ uint16_t f2bf(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ float bf2f(uint32_t b16) {
    return __builtin_bit_cast(float, b16 << 16);
}
// Two floats rounded to bf16 (round to nearest even, as f2bf) and packed,
// lo in bits 0..15: one v_cvt_pk_bf16_f32 for the pair.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
// The same bits from two separate conversions.  Only one float is live at a
// time, which suits kernels short of registers (the eight-wave dgrad
// instances measured about 5% slower with the paired form).
__device__ __forceinline__ uint32_t pack2_sep(float lo, float hi) {
    return static_cast<uint32_t>(f2bf(lo)) | (static_cast<uint32_t>(f2bf(hi)) << 16);
}
// The two bf16 values of a packed pair as floats.
__device__ __forceinline__ float lo_f(uint32_t pr) { return __builtin_bit_cast(float, pr << 16); }
__device__ __forceinline__ float hi_f(uint32_t pr) { return __builtin_bit_cast(float, pr & 0xffff0000u); }

// Chunk swizzles (chosen from LDS bank-conflict counter measurements on
// gfx950).  K-contiguous panels are [row][64 k] (128-byte rows, eight 16-byte
// chunks); chunk c of row r is stored at c ^ kswz(r), which keeps the 16-byte
// fragment reads (32 rows x 2 chunks per wave) conflict-free.  N-contiguous
// panels are [64 k][BN n]; chunk c of row k is stored at c ^ nswz(k), which
// keeps the 8-byte transpose reads conflict-free (it permutes 4-chunk blocks,
// so column offsets of 16 chunks stay additive).
__device__ __forceinline__ int kswz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int nswz(int k) { return (k & 3) << 2; }

// [row][64] K-contiguous panel: element offset of logical 16-byte chunk c (0..7) of `row`.
__device__ __forceinline__ int kc_off(int row, int c) {
    return row * BK + ((c ^ kswz(row)) << 3);
}
// [64][BN] N-contiguous panel: element offset of column n (multiple of 4) in row k.
template <int BN>
__device__ __forceinline__ int nc_off(int k, int n) {
    return k * BN + (((n >> 3) ^ nswz(k)) << 3) + (n & 7);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    asm volatile("" ::: "memory");
}
// Workgroup barrier for the copy pipeline.  It first waits for this wave's
// outstanding LDS operations: a fragment read issued before the barrier must
// have completed before another wave refills that stage slot with LDS-DMA.
// (Outstanding HBM->LDS copies are waited for explicitly with wait_vmcnt.)
__device__ __forceinline__ void block_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); the builtin keeps the compiler's count in step
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Wait states between the last MFMA and the first read of its accumulators.
// The compiler cannot count them where the read is inline assembly or where
// a branch skipped the last MFMA, so the epilogues issue them explicitly
// (24, more than a 16-pass MFMA needs).
__device__ __forceinline__ void mfma_drain() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}
template <typename T>
__device__ __forceinline__ const T* uni_ptr(const T* ptr) {
    const uint64_t v = reinterpret_cast<uint64_t>(ptr);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return reinterpret_cast<const T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// One wave-wide LDS-DMA load: every lane copies 16 bytes from base + voff
// (base wave-uniform, voff a per-lane 32-bit byte offset) to LDS byte address
// lds + 16 * lane (lds wave-uniform).  Issued from
// inline assembly so that the compiler does not add a conservative wait for
// all outstanding loads before every LDS read; the pipeline waits for the
// stage it needs explicitly (wait_vmcnt + barrier).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(uni_ptr(base)), "s"(uni(lds)) : "memory", "m0");
}
// The same copy marked non-temporal (low retention in the caches), for data
// read once per pass: the streamed weights of the streaming items, which
// would otherwise push out of L2 the token panels that every item re-reads.
__device__ __forceinline__ void dma16_nt(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(voff), "s"(uni_ptr(base)), "s"(uni(lds)) : "memory", "m0");
}
#pragma clang diagnostic pop

// Read one accumulator register in the epilogue.  The accumulators live in
// AGPRs; reading them one at a time where they are consumed keeps the
// compiler from copying all of them to VGPRs at once at the end of the K loop.
__device__ __forceinline__ float acc_rd(float a) {
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}
// SwiGLU of four outputs: gate and up accumulators q*4 .. q*4+3 of ga and
// ua, each rounded to bf16, then a = bf16(p * (g * sigmoid(slope * g) * u))
// (p = 1 without probabilities).  Returns the bf16 A, gate and up values as
// two packed pairs each.
__device__ __forceinline__ void swiglu4(const f32x16& ga, const f32x16& ua, int q, float slope, float pr,
                                        bool weighted, uint2& a_out, uint2& g_out, uint2& u_out) {
    uint32_t gp[2], up[2], ap[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        gp[h] = pack2(acc_rd(ga[q * 4 + 2 * h]), acc_rd(ga[q * 4 + 2 * h + 1]));
        up[h] = pack2(acc_rd(ua[q * 4 + 2 * h]), acc_rd(ua[q * 4 + 2 * h + 1]));
        float av[2];
#pragma unroll
        for (int y = 0; y < 2; ++y) {
            const float g = y ? hi_f(gp[h]) : lo_f(gp[h]);
            const float u = y ? hi_f(up[h]) : lo_f(up[h]);
            const float sg = g * __builtin_amdgcn_rcpf(1.0f + __expf(-(slope * g)));
            const float v = sg * u;
            av[y] = weighted ? pr * v : v;
        }
        ap[h] = pack2(av[0], av[1]);
    }
    a_out = make_uint2(ap[0], ap[1]);
    g_out = make_uint2(gp[0], gp[1]);
    u_out = make_uint2(up[0], up[1]);
}

template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
    return __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(GG_AS3(const_cast<T*>(p)))));
}

// Rows that do not fill a 256-row tile, if there are at most SMALL_M of them
// (every row of a small expert, or the tail of a large one), take the
// weight-streaming flavor: one work item per block of output columns covering
// all those rows, so each weight byte is read once for them.
constexpr int SMALL_M = 96;
constexpr int S_BLK = SMALL_M / 32;   // 32-row token blocks of a streaming item

// How an expert with m rows is split: full 256-row tiles, and the rows left
// over.  A remainder of at most SMALL_M rows (all the rows of a small expert,
// or the tail of a large one) is streamed; a larger remainder is one more,
// partial tile.
__device__ __forceinline__ int tile_rows_of(int m) {
    const int tail = m % 256;
    return (tail > 0 && tail <= SMALL_M) ? m - tail : m;     // rows covered by tiles
}
__device__ __forceinline__ int tiles_m_of(int m) { return (tile_rows_of(m) + 255) / 256; }
__device__ __forceinline__ bool streams_rows(int m) { return m > 0 && tile_rows_of(m) < m; }

// Per-expert work counts and their exclusive prefix sums in LDS, for both
// flavors: s_pre counts 256x256 tiles of the large experts, s_spre counts
// streaming items of the small ones.  Offsets are clamped into [0, M] so that
// bad offsets cannot index out of bounds.
template <int NT>
__device__ __forceinline__ void build_schedule(const int64_t* __restrict__ offsets, int E, int M,
                                               int tiles_n, int items_n, int* s_off, int* s_pre, int* s_spre) {
    const int tid = threadIdx.x;
    for (int e = tid; e <= E; e += NT) {
        int64_t o = offsets[e];
        o = o < 0 ? 0 : (o > M ? M : o);
        s_off[e] = static_cast<int>(o);
    }
    __syncthreads();
    if (tid < 64) {
        const int lane = tid;
        const int per = (E + 63) / 64;
        const int e0 = lane * per;
        const int e1 = min(E, e0 + per);
        auto rows = [&](int e) { return max(0, s_off[e + 1] - s_off[e]); };
        auto big = [&](int e) { return tiles_m_of(rows(e)) * tiles_n; };
        auto small = [&](int e) { return streams_rows(rows(e)) ? items_n : 0; };
        int sum = 0, ssum = 0;
        for (int e = e0; e < e1; ++e) {
            sum += big(e);
            ssum += small(e);
        }
        int incl = sum, sincl = ssum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            const int sv = __shfl_up(sincl, d, 64);
            if (lane >= d) {
                incl += v;
                sincl += sv;
            }
        }
        int run = incl - sum, srun = sincl - ssum;
        for (int e = e0; e < e1; ++e) {
            s_pre[e] = run;
            s_spre[e] = srun;
            run += big(e);
            srun += small(e);
        }
        if (lane == 63) {
            s_pre[E] = incl;
            s_spre[E] = sincl;
        }
    }
    __syncthreads();
}

// Largest e in [0, E-1] with s_pre[e] <= t (t < s_pre[E]); skips empty experts.
__device__ __forceinline__ int find_expert(const int* s_pre, int E, int t) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Tile geometry: a workgroup computes a 256 (token rows) x 256 (weight rows)
// output tile with 8 waves, two per SIMD.  Wave w belongs to group g = w / 4
// (token rows g*128 .. g*128+127) and owns 64 weight rows (w % 4); waves w and
// w + 4 share a SIMD.  The two groups alternate ("ping-pong"): while one
// group issues its MFMAs for a K stage, the other reads its fragments for
// that stage from LDS and issues the HBM->LDS copies, and a barrier swaps the
// roles, so the matrix pipe of every SIMD always has a wave feeding it.
template <int V> struct GrpTag { static constexpr int value = V; };
// f(GrpTag<0>{}), ..., f(GrpTag<N - 1>{}): a loop over compile-time indices.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(GrpTag<I>{});
        static_for<N, I + 1>(f);
    }
}
constexpr int TBM = 256, TBN = 256, NWAVES = 8, NTHREADS = NWAVES * 64, NSTAGE = 2;
constexpr int WROWS = 128, WCOLS = 64, FM = WROWS / 32, FN = WCOLS / 32;
constexpr int A_STAGE = TBM * BK, B_STAGE = TBN * BK;          // elements per stage
constexpr int A_PW = A_STAGE * 2 / 1024 / NWAVES;               // 1 KiB DMA instructions per wave
constexpr int B_PW = B_STAGE * 2 / 1024 / NWAVES;
constexpr int LPS = A_PW + B_PW;                                // per wave per stage
static_assert(A_PW * NWAVES * 1024 == A_STAGE * 2 && B_PW * NWAVES * 1024 == B_STAGE * 2, "DMA split");
// The streaming flavor's ring (4 stages of 192 weight rows + SMALL_M token
// rows, 64 k each) lays its stages over the same LDS as the tile stages.
constexpr int S_RING_EL = 4 * (192 + SMALL_M) * BK;
constexpr int LDS_BUF_EL = S_RING_EL > NSTAGE * (A_STAGE + B_STAGE) ? S_RING_EL : NSTAGE * (A_STAGE + B_STAGE);

// EXT selects the activation options (QuickGeGLU slope, per-row weights, dp
// partial sums).  Without it they fold to plain SwiGLU, so the plain
// instantiations carry none of their registers.
template <bool W_KN, int EPI, bool EXT>
__global__ __launch_bounds__(NTHREADS)
void grouped_gemm_kernel(const GemmParams p) {
    // bf16 pair packing for the epilogues: separate conversions in the dgrad
    // instances (transposed weights), which are short of registers
    auto pk = [](float lo, float hi) -> uint32_t {
        if constexpr (W_KN) return pack2_sep(lo, hi);
        else return pack2(lo, hi);
    };
    const float slope = EXT ? p.slope : 1.0f;
    const float* const probs = EXT ? p.probs : nullptr;
    float* const dp_part = EXT ? p.dp_part : nullptr;
    // Operand stages: NSTAGE token panels, then NSTAGE weight panels (the
    // streaming flavor lays its own stages over the same bytes).
    __shared__ __attribute__((aligned(1024))) uint16_t s_buf[LDS_BUF_EL];
    __shared__ int s_off[GG_KMAX_EXPERTS + 1];
    __shared__ int s_pre[GG_KMAX_EXPERTS + 1];
    __shared__ int s_spre[GG_KMAX_EXPERTS + 1];
    auto s_a = [&](int st) -> uint16_t* { return s_buf + st * A_STAGE; };
    auto s_b = [&](int st) -> uint16_t* { return s_buf + NSTAGE * A_STAGE + st * B_STAGE; };

    const int E = p.E, M = p.M, K = p.K, N = p.N;
    constexpr int TILE_COLS = (EPI == EPI_SWIGLU) ? TBN / 2 : TBN;
    const int tiles_n = (N + TILE_COLS - 1) / TILE_COLS;
    // streaming flavor: an item is the streamed rows of one expert x S_COLS output
    // columns (192 weight rows: for SwiGLU 96 gate rows and the matching 96 up rows)
    constexpr int S_ROWS = 192;                                   // weight rows per item
    constexpr int S_COLS = (EPI == EPI_SWIGLU) ? S_ROWS / 2 : S_ROWS;
    const int items_n = (N + S_COLS - 1) / S_COLS;
    static_assert(TBM == 256, "tile_rows_of assumes 256-row tiles");
    build_schedule<NTHREADS>(p.offsets, E, M, tiles_n, items_n, s_off, s_pre, s_spre);
    const int n_items = uni(s_spre[E]);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uni(tid >> 6);
    const int grp = wave >> 2;          // 0: token rows 0..127, 1: 128..255
    const int wq = wave & 3;            // weight-row block
    const int kiters = (K + BK - 1) / BK;
    const bool k_tail = (K % BK) != 0;
    const uint32_t a_lds0 = lds_addr(s_a(0)) + wave * A_PW * 1024;
    const uint32_t b_lds0 = lds_addr(s_b(0)) + wave * B_PW * 1024;

    // Workgroups are dealt round-robin over the 8 XCDs; give the workgroups of
    // one XCD consecutive tiles so that tiles sharing panels share an L2.
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int slot = (G % 8 == 0) ? (b & 7) * (G >> 3) + (b >> 3) : b;
    // When the streaming items fit into the grid twice over, each is split into
    // two halves of S_ROWS / 2 weight rows (three compute waves), so that no
    // workgroup takes a whole item while others take none.  A row's arithmetic
    // is the same either way.
    const int s_sh = (2 * n_items <= G) ? 1 : 0;   // log2 of the halves per item
    const int n_stream = n_items << s_sh;

    // ---- per-tile state (wave-uniform values live in SGPRs)
    int row0 = 0, row_end = 0, col0 = 0;
    const uint16_t* a_base = p.act;   // first row of the tile
    const uint16_t* w_base = p.w;     // this expert's weight matrix
    uint32_t a_voff[A_PW];            // byte offset of the chunk this lane moves (k0 = 0)
    uint32_t b_voff[B_PW];
    int a_kc[A_PW];                   // k offset of the chunk (K-contiguous)
    int b_kc[B_PW];                   // k offset (K-contiguous) / panel row (N-contiguous)

    auto setup_tile = [&](int t) {   // t: index among the 256x256 tiles
        const int e = uni(find_expert(s_pre, E, t));
        const int local = t - uni(s_pre[e]);
        const int rb = uni(s_off[e]);
        row_end = uni(s_off[e + 1]);
        const int tiles_m = tiles_m_of(row_end - rb);
        row0 = rb + (local % tiles_m) * TBM;
        col0 = (local / tiles_m) * TILE_COLS;
        a_base = p.act + static_cast<int64_t>(row0) * K;
        w_base = p.w + static_cast<int64_t>(e) * p.w_expert_stride;
        const int rows = row_end - row0;
#pragma unroll
        for (int i = 0; i < A_PW; ++i) {
            const int pos = (wave * A_PW + i) * 64 + lane;   // 16-byte chunk slot in the stage
            const int r = pos >> 3;
            const int c = (pos & 7) ^ kswz(r);                 // logical chunk stored there
            a_voff[i] = static_cast<uint32_t>((min(r, rows - 1) * K + c * 8) * 2);
            a_kc[i] = c * 8;
        }
#pragma unroll
        for (int i = 0; i < B_PW; ++i) {
            const int pos = (wave * B_PW + i) * 64 + lane;
            if constexpr (!W_KN) {
                const int r = pos >> 3;
                const int c = (pos & 7) ^ kswz(r);
                int wrow;
                if constexpr (EPI == EPI_SWIGLU) {
                    const int half = r / (TBN / 2);
                    wrow = min(col0 + r % (TBN / 2), N - 1) + half * p.up_off;
                } else {
                    wrow = min(col0 + r, N - 1);
                }
                b_voff[i] = static_cast<uint32_t>((wrow * p.ldw + c * 8) * 2);
                b_kc[i] = c * 8;
            } else {
                constexpr int CPR = TBN / 8;                   // chunks per panel row
                const int k = pos / CPR;
                const int c = (pos % CPR) ^ nswz(k);
                b_voff[i] = static_cast<uint32_t>((k * p.ldw + min(col0 + c * 8, N - 8)) * 2);
                b_kc[i] = k;
            }
        }
    };

    // Copy K stage kt of both panels into its LDS slot (this wave's share).
    auto issue = [&](int kt) {
        const int stage = kt % NSTAGE;
        const int k0 = kt * BK;
        const bool tail = k_tail && kt == kiters - 1;
#pragma unroll
        for (int i = 0; i < A_PW; ++i) {
            const uint32_t lds = a_lds0 + stage * (A_STAGE * 2) + i * 1024;
            if (!tail) {
                dma16(a_base + k0, a_voff[i], lds);
            } else {
                // chunks at k >= K re-read k = 0 of the same row (in bounds); zeroed later
                const uint32_t v = (k0 + a_kc[i] < K) ? a_voff[i] + k0 * 2 : a_voff[i] - a_kc[i] * 2;
                dma16(a_base, v, lds);
            }
        }
#pragma unroll
        for (int i = 0; i < B_PW; ++i) {
            const uint32_t lds = b_lds0 + stage * (B_STAGE * 2) + i * 1024;
            if constexpr (!W_KN) {
                if (!tail) {
                    dma16(w_base + k0, b_voff[i], lds);
                } else {
                    const uint32_t v = (k0 + b_kc[i] < K) ? b_voff[i] + k0 * 2 : b_voff[i] - b_kc[i] * 2;
                    dma16(w_base, v, lds);
                }
            } else {
                if (!tail) {
                    dma16(w_base + static_cast<int64_t>(k0) * p.ldw, b_voff[i], lds);
                } else {
                    // rows >= K re-read row K-1 (in bounds); zeroed later
                    const int row = min(k0 + b_kc[i], K - 1);
                    const uint32_t v = b_voff[i] + static_cast<uint32_t>((row - b_kc[i]) * p.ldw * 2);
                    dma16(w_base, v, lds);
                }
            }
        }
    };

    // Wait until this wave's copies of a stage have landed, given how many later
    // stages it has in flight.
    auto wait_stage = [&](int newer) {
        if (newer <= 0) wait_vmcnt<0>();
        else wait_vmcnt<LPS>();
    };

    // Zero the K positions >= K of a stage (only when K % BK != 0, last stage).
    auto zero_tail = [&](int kt) {
        const int stage = kt % NSTAGE;
        const int k0 = kt * BK;
        for (int idx = tid; idx < TBM * 8; idx += NTHREADS) {
            const int r = idx >> 3, c = idx & 7;
            if (k0 + c * 8 >= K)
                *reinterpret_cast<uint4*>(s_a(stage) + kc_off(r, c)) = make_uint4(0, 0, 0, 0);
        }
        if constexpr (!W_KN) {
            for (int idx = tid; idx < TBN * 8; idx += NTHREADS) {
                const int r = idx >> 3, c = idx & 7;
                if (k0 + c * 8 >= K)
                    *reinterpret_cast<uint4*>(s_b(stage) + kc_off(r, c)) = make_uint4(0, 0, 0, 0);
            }
        } else {
            for (int idx = tid; idx < BK * TBN / 8; idx += NTHREADS) {
                const int k = idx / (TBN / 8), c = idx % (TBN / 8);
                if (k0 + k >= K)
                    *reinterpret_cast<uint4*>(s_b(stage) + k * TBN + c * 8) = make_uint4(0, 0, 0, 0);
            }
        }
    };

    // column (relative to the tile) of local 16-byte chunk c (0..7) of a wave's
    // 64 output columns: fragment j = c / 4 sits in tile half j
    auto wcol = [&](int c) -> int { return (c >> 2) * (TBN / 2) + wq * 32 + (c & 3) * 8; };

    // first weight-panel row (K-contiguous) or column (N-contiguous) of fragment j
    auto wfrag = [&](int j) -> int {
        if constexpr (EPI == EPI_SWIGLU) {
            return j == 0 ? wq * 32 : TBN / 2 + wq * 32;     // gate rows, matching up rows
        } else {
            return j * (TBN / 2) + wq * 32;   // 32 columns in each half of the tile
        }
    };

    bf16x8 fa[2][FM], fb[2][FN];
    // fragments of half-stage h (K elements h*32 .. h*32+31): stage h/2, half h%2
    auto load_frags = [&](int h) {
        const uint16_t* sa = s_a((h >> 1) % NSTAGE);
        const uint16_t* sb = s_b((h >> 1) % NSTAGE);
        const int half = h & 1;
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
            const int ch = half * 4 + ss * 2 + (lane >> 5);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = grp * WROWS + i * 32 + (lane & 31);
                fa[ss][i] = *reinterpret_cast<const bf16x8*>(sa + kc_off(r, ch));
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if constexpr (!W_KN) {
                    const int r = wfrag(j) + (lane & 31);
                    fb[ss][j] = *reinterpret_cast<const bf16x8*>(sb + kc_off(r, ch));
                } else {
                    // lane 16g + 4s + q supplies (k = kb + s, n = nb + 4q) and receives
                    // column nb + (lane & 15), rows kb .. kb+3 (ds_read_b64_tr_b16).
                    const int g = lane >> 4;
                    const int kb = half * HK + ss * 16 + 8 * (g >> 1) + ((lane >> 2) & 3);
                    const int n = wfrag(j) + 16 * (g & 1) + 4 * (lane & 3);
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        reinterpret_cast<__attribute__((address_space(3))) i16x4*>(
                            GG_AS3(sb + nc_off<TBN>(kb, n))));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        reinterpret_cast<__attribute__((address_space(3))) i16x4*>(
                            GG_AS3(sb + nc_off<TBN>(kb + 4, n))));
                    const __attribute__((ext_vector_type(8))) short v8 =
                        __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    fb[ss][j] = __builtin_bit_cast(bf16x8, v8);
                }
            }
        }
    };

    // one k16 step ss (0, 1) of half-stage h into fa[ss], fb[ss] (K-contiguous
    // weights; the pipelined loop below)
    auto load_step = [&](int h, int ss) {
        const uint16_t* sa = s_a((h >> 1) % NSTAGE);
        const uint16_t* sb = s_b((h >> 1) % NSTAGE);
        const int ch = (h & 1) * 4 + ss * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int r = grp * WROWS + i * 32 + (lane & 31);
            fa[ss][i] = *reinterpret_cast<const bf16x8*>(sa + kc_off(r, ch));
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int r = wfrag(j) + (lane & 31);
            fb[ss][j] = *reinterpret_cast<const bf16x8*>(sb + kc_off(r, ch));
        }
    };
    f32x16 acc[FM][FN];
    auto mma_step = [&](int ss) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ss][j], fa[ss][i], acc[i][j], 0, 0, 0);
    };
    auto mma = [&]() {
#pragma unroll
        for (int ss = 0; ss < 2; ++ss)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ss][j], fa[ss][i], acc[i][j], 0, 0, 0);
    };

    // ---- streaming flavor (small experts): weight streaming.  Workgroups take
    // items round-robin.  Per 64-wide K stage the weight panel holds S_ROWS rows
    // (K-contiguous weights; for SwiGLU wave w's 32 rows are 16 gate rows then
    // the matching 16 up rows) or S_ROWS columns (transposed weights), and the
    // token panel SMALL_M rows (rows past the expert's end repeat its last row).
    // A 4-stage ring of 36 KiB runs continuously across the items, so the
    // copies of the next item are in flight while the current one finishes.
    // Waves w < S_WAVES compute 32 weight rows each against one to S_BLK
    // 32-row token blocks and store the results; the other two waves issue every
    // copy, so a copy wave's vmcnt counts copies only (vmcnt retires in
    // order: a store queued among the copies would be waited for with them).
    constexpr int SX_EL = SMALL_M * BK;
    constexpr int S_NST = 4, SW_EL = S_ROWS * BK, S_EL = SW_EL + SX_EL;
    constexpr int S_WAVES = S_ROWS / 32;              // waves with weight rows to compute
    constexpr int S_CWAVES = NWAVES - S_WAVES;        // copy waves
    constexpr int SW_PW = SW_EL * 2 / 1024 / S_CWAVES; // weight-panel copies per copy wave per stage
    constexpr int SX_PW = SX_EL * 2 / 1024 / S_CWAVES; // token-panel copies per copy wave per stage
    constexpr int LPS_S = SW_PW + SX_PW;
    static_assert(SW_PW * S_CWAVES * 1024 == SW_EL * 2 && SX_PW * S_CWAVES * 1024 == SX_EL * 2, "copy split");
    static_assert(3 * LPS_S < 64, "vmcnt range");
    constexpr int S_CPR = S_ROWS / 8;                 // 16-byte chunks per transposed-panel row
    // transposed panels [64 k][S_ROWS n]: chunk c of row k at c ^ (2 * (k & 3)),
    // which keeps every chunk inside its aligned group of 8
    auto snc_off = [](int k, int n) { return k * S_ROWS + (((n >> 3) ^ ((k & 3) << 1)) << 3) + (n & 7); };
    static_assert(S_NST * S_EL <= LDS_BUF_EL, "streaming stages fit in LDS");
    struct SItem { int e, row0, rows, col0; };
    const int s_aw = S_WAVES >> s_sh;            // compute waves with rows in an item
    auto stream_items = [&](int t0) -> int {
        const int n_my = (n_stream - t0 + G - 1) / G;
        const int nq = n_my * kiters;
        const uint32_t s_lds0 = lds_addr(s_buf);
        auto item_of = [&](int i) -> SItem {
            const int t = t0 + i * G;
            const int tf = t >> s_sh;                // whole item
            SItem it;
            it.e = uni(find_expert(s_spre, E, tf));
            const int rb = uni(s_off[it.e]), re = uni(s_off[it.e + 1]);
            it.row0 = rb + tile_rows_of(re - rb);   // the rows the tiles leave
            it.rows = re - it.row0;
            it.col0 = (tf - uni(s_spre[it.e])) * S_COLS + (t & s_sh) * (S_COLS / 2);
            return it;
        };
        auto issue_s = [&](const SItem& it, int kt, int slot_i) {
            if (wave < S_WAVES) return;
            const int cw = wave - S_WAVES;
            const int k0 = kt * BK;
            const uint32_t base = s_lds0 + slot_i * (S_EL * 2);
            const uint16_t* wb = p.w + static_cast<int64_t>(it.e) * p.w_expert_stride;
#pragma unroll
            for (int i = 0; i < SW_PW; ++i) {
                const int pos = (cw * SW_PW + i) * 64 + lane;
                uint32_t voff;
                // a half item's unused panel half re-reads its used half (L2
                // hits), so every stage issues the same number of copies
                if constexpr (!W_KN) {
                    const int r = pos >> 3;
                    const int c = (pos & 7) ^ kswz(r);
                    const int rr = (s_sh && r >= S_ROWS / 2) ? r - S_ROWS / 2 : r;
                    int wrow;
                    if constexpr (EPI == EPI_SWIGLU) {
                        const int q = rr & 31;
                        wrow = min(it.col0 + (rr >> 5) * 16 + (q & 15), N - 1) + (q >= 16 ? p.up_off : 0);
                    } else {
                        wrow = min(it.col0 + rr, N - 1);
                    }
                    voff = static_cast<uint32_t>((wrow * p.ldw + min(k0 + c * 8, K - 8)) * 2);
                } else {
                    const int kr = pos / S_CPR;
                    const int c = (pos % S_CPR) ^ ((kr & 3) << 1);
                    const int cc = (s_sh && c >= S_CPR / 2) ? c - S_CPR / 2 : c;
                    voff = static_cast<uint32_t>((min(k0 + kr, K - 1) * p.ldw + min(it.col0 + cc * 8, N - 8)) * 2);
                }
                dma16_nt(wb, voff, base + (cw * SW_PW + i) * 1024);
            }
            const uint16_t* xb = p.act + static_cast<int64_t>(it.row0) * K;
#pragma unroll
            for (int i = 0; i < SX_PW; ++i) {
                const int pos = (cw * SX_PW + i) * 64 + lane;
                const int r = pos >> 3;
                const int c = (pos & 7) ^ kswz(r);
                const uint32_t xoff = static_cast<uint32_t>((min(r, it.rows - 1) * K + min(k0 + c * 8, K - 8)) * 2);
                dma16(xb, xoff, base + SW_EL * 2 + (cw * SX_PW + i) * 1024);
            }
        };
        f32x16 sacc[S_BLK];
        auto szero = [&]() {
#pragma unroll
            for (int b = 0; b < S_BLK; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) sacc[b][v] = 0.f;
        };
        // K positions >= K (last stage only) are zeroed in the fragments, so
        // whatever the copies left there adds nothing (the tile flavor adds the
        // same zero products).  Every fragment read of the stage is issued
        // before its MFMAs, in two k32 halves (which bounds the fragment
        // registers), so the LDS latency is paid twice per stage; the token
        // fragments of all S_BLK blocks are read whatever nblk is (the panel
        // always holds SMALL_M rows), which keeps the reads independent.
        auto s_mma = [&](int slot_i, int kt, int nblk) {
            const uint16_t* sw = s_buf + slot_i * S_EL;
            const uint16_t* sx = sw + SW_EL;
            constexpr int NJ = BK / 16, NH = NJ / 2;
            const bool last = k_tail && kt == kiters - 1;   // uniform: only the last stage has a tail
#pragma unroll
            for (int h = 0; h < 2; ++h) {   // two k32 halves: bounds the fragment registers
                bf16x8 wf[NH], xf[NH][S_BLK];
#pragma unroll
                for (int jj = 0; jj < NH; ++jj) {
                    const int j = h * NH + jj;
                    const int ch = 2 * j + (lane >> 5);
                    if constexpr (!W_KN) {
                        wf[jj] = *reinterpret_cast<const bf16x8*>(sw + kc_off(wave * 32 + (lane & 31), ch));
                    } else {
                        const int g = lane >> 4;
                        const int kb = j * 16 + 8 * (g >> 1) + ((lane >> 2) & 3);
                        const int n = wave * 32 + 16 * (g & 1) + 4 * (lane & 3);
                        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            reinterpret_cast<__attribute__((address_space(3))) i16x4*>(GG_AS3(sw + snc_off(kb, n))));
                        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            reinterpret_cast<__attribute__((address_space(3))) i16x4*>(GG_AS3(sw + snc_off(kb + 4, n))));
                        wf[jj] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    }
#pragma unroll
                    for (int b = 0; b < S_BLK; ++b)
                        xf[jj][b] = *reinterpret_cast<const bf16x8*>(sx + kc_off(b * 32 + (lane & 31), ch));
                }
                if (last) {
#pragma unroll
                    for (int jj = 0; jj < NH; ++jj) {
                        if (kt * BK + (h * NH + jj) * 16 + 8 * (lane >> 5) >= K) {
                            const bf16x8 z = {};
                            wf[jj] = z;
#pragma unroll
                            for (int b = 0; b < S_BLK; ++b) xf[jj][b] = z;
                        }
                    }
                }
#pragma unroll
                for (int jj = 0; jj < NH; ++jj) {
                    sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[jj], xf[jj][0], sacc[0], 0, 0, 0);
#pragma unroll
                    for (int b = 1; b < S_BLK; ++b)
                        if (b < nblk) sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[jj], xf[jj][b], sacc[b], 0, 0, 0);
                }
            }
        };

        // Item epilogue, staged through the ring slot of the item's last stage:
        // every wave has finished reading it at the first barrier below, and
        // the copy waves refill it only after the next stage's barrier.  Per
        // 32-row token block the compute waves write their results into a
        // [32][SC] bf16 array (one pad chunk per row), then store whole row
        // segments with 16-byte stores: scattered 8-byte stores from the
        // accumulator layout cost several times the write requests per byte.
        // The derivative variant first copies the block's saved gate|up rows
        // into the array with LDS-DMA and overwrites them in place.
        // Lane holds token (lane & 31) of block b and, for register v, panel row
        // 8*(v/4) + 4*(lane/32) + v%4 of the wave's 32 rows.
        constexpr int SC = (EPI == EPI_SWIGLU) ? 3 * S_COLS : (EPI == EPI_DSWIGLU ? 2 * S_COLS : S_COLS);
        constexpr int SCH = SC / 8;             // 16-byte chunks per staged row
        constexpr int SLD = SC + 8;             // staged row stride in elements
        constexpr int S_STG_DMA = (32 * (SCH + 1) + 63) / 64;   // derivative: DMA instructions per block
        static_assert(SC % 8 == 0 && S_STG_DMA * 1024 <= S_EL * 2, "staging fits in a ring slot");
        auto s_epilogue = [&](const SItem& it, int nblk, int slot_i) {
            uint16_t* stg = s_buf + slot_i * S_EL;
            const bool cwave = wave < S_WAVES;  // stores
            const bool awave = wave < s_aw;     // holds results of this item
            const int col_end = min(N, it.col0 + (S_COLS >> s_sh));
            block_barrier();                    // every wave is done with the slot
            if (awave) mfma_drain();
#pragma unroll
            for (int b = 0; b < S_BLK; ++b) {
                if (b >= nblk) break;           // nblk is uniform over the workgroup
                const int tok = b * 32 + (lane & 31);
                const bool rv = tok < it.rows;
                const int64_t grow = it.row0 + tok;
                const int r = lane & 31;
                if constexpr (EPI == EPI_DSWIGLU) {
                    // saved H1 of the block: gate columns then up columns of each row;
                    // slots past the rows or columns re-read in-bounds data
                    if (cwave) {
                        const uint16_t* hb = p.aux + static_cast<int64_t>(it.row0) * (2 * N);
                        const uint32_t stg_lds = lds_addr(stg);
                        for (int ins = wave; ins < S_STG_DMA; ins += S_WAVES) {
                            const int sl = ins * 64 + lane;
                            const int sr = min(sl / (SCH + 1), 31);
                            int sc = sl % (SCH + 1);
                            if (sc == SCH) sc = 0;
                            const int arr = sc / (SCH / 2), cc = sc % (SCH / 2);
                            const int row = min(b * 32 + sr, it.rows - 1);
                            const int f = min(it.col0 + cc * 8, N - 8);
                            dma16(hb, static_cast<uint32_t>((row * 2 * N + arr * N + f) * 2), stg_lds + ins * 1024);
                        }
                        wait_vmcnt<0>();
                    }
                    block_barrier();
                }
                if (awave) {
                    if constexpr (EPI == EPI_STORE) {
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int cl = wave * 32 + 8 * g + 4 * (lane >> 5);
                            *reinterpret_cast<uint2*>(stg + r * SLD + cl) =
                                make_uint2(pk(acc_rd(sacc[b][4 * g]), acc_rd(sacc[b][4 * g + 1])),
                                           pk(acc_rd(sacc[b][4 * g + 2]), acc_rd(sacc[b][4 * g + 3])));
                        }
                    } else if constexpr (EPI == EPI_SWIGLU) {
                        const float pr = (probs && rv) ? probs[grow] : 1.0f;
#pragma unroll
                        for (int g = 0; g < 2; ++g) {
                            const int fl = wave * 16 + 8 * g + 4 * (lane >> 5);
                            uint32_t gp[2], up[2], ap[2];   // bf16 pairs
#pragma unroll
                            for (int h = 0; h < 2; ++h) {
                                gp[h] = pack2(acc_rd(sacc[b][4 * g + 2 * h]), acc_rd(sacc[b][4 * g + 2 * h + 1]));
                                up[h] = pack2(acc_rd(sacc[b][4 * g + 8 + 2 * h]), acc_rd(sacc[b][4 * g + 8 + 2 * h + 1]));
                                float av[2];
#pragma unroll
                                for (int y = 0; y < 2; ++y) {
                                    const float gg = y ? hi_f(gp[h]) : lo_f(gp[h]);
                                    const float uu = y ? hi_f(up[h]) : lo_f(up[h]);
                                    const float v = gg * __builtin_amdgcn_rcpf(1.0f + __expf(-(slope * gg))) * uu;
                                    av[y] = probs ? pr * v : v;
                                }
                                ap[h] = pack2(av[0], av[1]);
                            }
                            uint16_t* sr = stg + r * SLD + fl;
                            *reinterpret_cast<uint2*>(sr) = make_uint2(ap[0], ap[1]);
                            *reinterpret_cast<uint2*>(sr + S_COLS) = make_uint2(gp[0], gp[1]);
                            *reinterpret_cast<uint2*>(sr + 2 * S_COLS) = make_uint2(up[0], up[1]);
                        }
                    } else {
                        const float pr = (probs && rv) ? probs[grow] : 1.0f;
                        float dps = 0.0f;   // this lane's share of dp over the wave's 32 columns
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int cl = wave * 32 + 8 * g + 4 * (lane >> 5);
                            const bool fv = rv && it.col0 + cl < N;
                            uint16_t* sg = stg + r * SLD + cl;
                            const uint2 hg = *reinterpret_cast<const uint2*>(sg);
                            const uint2 hu = *reinterpret_cast<const uint2*>(sg + S_COLS);
                            const uint32_t gw[2] = {hg.x, hg.y};
                            const uint32_t uw[2] = {hu.x, hu.y};
                            const uint32_t dw[2] = {pk(acc_rd(sacc[b][4 * g]), acc_rd(sacc[b][4 * g + 1])),
                                                    pk(acc_rd(sacc[b][4 * g + 2]), acc_rd(sacc[b][4 * g + 3]))};
                            float dg[4], du[4];
#pragma unroll
                            for (int x = 0; x < 4; ++x) {
                                const float gg = (x & 1) ? hi_f(gw[x >> 1]) : lo_f(gw[x >> 1]);
                                const float uu = (x & 1) ? hi_f(uw[x >> 1]) : lo_f(uw[x >> 1]);
                                const float da = (x & 1) ? hi_f(dw[x >> 1]) : lo_f(dw[x >> 1]);
                                const float sgm = __builtin_amdgcn_rcpf(1.0f + __expf(-(slope * gg)));
                                const float dap = probs ? pr * da : da;
                                dg[x] = dap * uu * sgm * (1.0f + slope * gg * (1.0f - sgm));
                                du[x] = dap * gg * sgm;
                                if (fv) dps += da * (gg * sgm * uu);
                            }
                            *reinterpret_cast<uint2*>(sg) = make_uint2(pk(dg[0], dg[1]), pk(dg[2], dg[3]));
                            *reinterpret_cast<uint2*>(sg + S_COLS) = make_uint2(pk(du[0], du[1]), pk(du[2], du[3]));
                        }
                        if (dp_part) {
                            // lanes l and l + 32 hold the two halves of the row's 32 columns
                            const float tot = dps + __shfl_xor(dps, 32, 64);
                            const int c0 = it.col0 + wave * 32;
                            if (lane < 32 && rv && c0 < N) dp_part[grow * p.dp_ld + c0 / 32] = tot;
                        }
                    }
                }
                block_barrier();
                if (cwave) {
                    for (int idx = wave * 64 + lane; idx < 32 * SCH; idx += S_WAVES * 64) {
                        const int sr = idx / SCH, sc = idx % SCH;
                        const int row = b * 32 + sr;
                        const uint4 v = *reinterpret_cast<const uint4*>(stg + sr * SLD + sc * 8);
                        if (row < it.rows) {
                            const int64_t orow = it.row0 + row;
                            if constexpr (EPI == EPI_STORE) {
                                const int col = it.col0 + sc * 8;
                                if (col < col_end) *reinterpret_cast<uint4*>(p.out0 + orow * N + col) = v;
                            } else if constexpr (EPI == EPI_SWIGLU) {
                                const int arr = sc / (SCH / 3), f = it.col0 + (sc % (SCH / 3)) * 8;
                                if (f < col_end) {
                                    if (arr == 0) *reinterpret_cast<uint4*>(p.out0 + orow * N + f) = v;
                                    else if (p.out1)
                                        *reinterpret_cast<uint4*>(p.out1 + orow * (2 * N) + (arr - 1) * N + f) = v;
                                }
                            } else {
                                const int arr = sc / (SCH / 2), f = it.col0 + (sc % (SCH / 2)) * 8;
                                if (f < col_end) *reinterpret_cast<uint4*>(p.out0 + orow * (2 * N) + arr * N + f) = v;
                            }
                        }
                    }
                }
                if (b + 1 < nblk) block_barrier();   // the next block overwrites the array
            }
        };

        SItem it_d = item_of(0);   // copy cursor
        int d_i = 0, d_kt = 0;
        auto advance = [&]() {
            if (++d_kt == kiters) {
                d_kt = 0;
                if (++d_i < n_my) it_d = item_of(d_i);
            }
        };
        for (int q = 0; q < S_NST - 1; ++q)
            if (q < nq) {
                issue_s(it_d, d_kt, q);
                advance();
            }
        // One pass per item, with the K stages inside.  Compute waves and copy
        // waves run separate copies of the item loop with the same barrier
        // sequence (one per stage, then the epilogue's), so that only MFMA
        // results cross the compute loop's back edge (the accumulators stay in
        // AGPRs) and neither role keeps the other's state live.
        if (wave < S_WAVES) {
            for (int i = 0, q = 0; i < n_my; ++i, q += kiters) {
                const SItem it_c = item_of(i);
                const int nblk = (it_c.rows + 31) / 32;
                if (wave < s_aw) {
                    szero();
                    for (int kt = 0; kt < kiters; ++kt) {
                        block_barrier();   // stage q + kt has landed
                        s_mma((q + kt) % S_NST, kt, nblk);
                    }
                } else {   // no rows in a half item
                    for (int kt = 0; kt < kiters; ++kt) block_barrier();
                }
                s_epilogue(it_c, nblk, (q + kiters - 1) % S_NST);
            }
        } else {
            for (int i = 0, q = 0; i < n_my; ++i) {
                for (int kt = 0; kt < kiters; ++kt, ++q) {
                    // wait for stage q (up to S_NST - 2 later stages stay in flight);
                    // the barrier publishes it to the compute waves
                    const int newer = min(S_NST - 2, nq - 1 - q);
                    if (newer >= 2) wait_vmcnt<2 * LPS_S>();
                    else if (newer == 1) wait_vmcnt<LPS_S>();
                    else wait_vmcnt<0>();
                    block_barrier();
                    // every wave has read stage q-1 (the barrier waited for the
                    // reads): refill its slot
                    if (q + S_NST - 1 < nq) {
                        issue_s(it_d, d_kt, (q + S_NST - 1) % S_NST);
                        advance();
                    }
                }
                // the epilogue's barriers (its work belongs to the compute waves)
                const SItem it_e = item_of(i);
                s_epilogue(it_e, (it_e.rows + 31) / 32, (q - 1) % S_NST);
            }
        }
        // the tile loop reuses the LDS
        block_barrier();
        return t0 + n_my * G;
    };

    // ---- streaming flavor first (work items [0, n_stream)), then the tiles
    int t = slot;
    if (t < n_stream) t = uni(stream_items(t));
    const int n_tiles = uni(s_pre[E]);
    for (int tt = t - n_stream; tt < n_tiles; tt += G) {
        setup_tile(tt);
#pragma unroll
        for (int s = 0; s < NSTAGE; ++s)
            if (s < kiters) issue(s);
        wait_stage(min(NSTAGE - 1, kiters - 1));
        block_barrier();
        if (k_tail && kiters == 1) {
            zero_tail(0);
            __syncthreads();
        }
        // Phases are half-stages.  The two groups run the same barrier sequence
        // (two per phase) on separate code paths so that each keeps its
        // fragments in fixed registers.
        const int nh = 2 * kiters;
        auto mid_phase = [&](int h) {
            // half h+1 starts a new stage: it must have landed (nothing newer is in flight)
            if ((h & 1) && h + 1 < nh) wait_stage(0);
            block_barrier();
            if (h & 1) {
                // stage h/2 is consumed by both groups: refill its slot
                if ((h >> 1) + NSTAGE < kiters) issue((h >> 1) + NSTAGE);
                if (k_tail && (h + 1) / 2 == kiters - 1 && h + 1 < nh) {
                    zero_tail(kiters - 1);
                    __syncthreads();
                }
            }
        };
        auto run_group = [&](auto gtag) {
        constexpr int GRP = decltype(gtag)::value;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
        if constexpr (!W_KN) {
            // K-contiguous weights: every wave pipelines its own k16 steps (the
            // fragments of the next step are read while this step's MFMAs issue;
            // the other wave on the SIMD covers the wait), one barrier per stage.
            // Measured faster than the ping-pong below for these panels.
            load_step(0, 0);
            for (int h = 0; h < nh; ++h) {
                __builtin_amdgcn_sched_barrier(0);
                load_step(h, 1);
                __builtin_amdgcn_sched_barrier(0);
                mma_step(0);
                __builtin_amdgcn_sched_barrier(0);
                if (h + 1 < nh) {
                    if (h & 1) {
                        // half h+1 starts stage (h+1)/2: it has landed (each wave waits
                        // for its own copies, the barrier for everyone's), and every
                        // wave has finished reading stage h/2 (the barrier first waits
                        // for outstanding LDS reads), so its slot is refilled
                        wait_stage(0);
                        block_barrier();
                        if ((h >> 1) + NSTAGE < kiters) issue((h >> 1) + NSTAGE);
                        if (k_tail && (h + 1) / 2 == kiters - 1) {
                            zero_tail(kiters - 1);
                            __syncthreads();
                        }
                    }
                    load_step(h + 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                mma_step(1);
            }
            // the epilogue stages results in the stage slots: every wave's last
            // fragment reads must have completed first
            block_barrier();
        } else if constexpr (GRP == 0) {
            // transposed weights (ds_read_b64_tr_b16 fragments): ping-pong, the
            // two groups alternate reading and computing half-stages
            load_frags(0);
            for (int h = 0; h < nh; ++h) {
                __builtin_amdgcn_sched_barrier(0);
                mma();                                   // phase 0: compute half h
                __builtin_amdgcn_sched_barrier(0);
                mid_phase(h);
                if (h + 1 < nh) load_frags(h + 1);       // phase 1: read half h+1
                __builtin_amdgcn_sched_barrier(0);
                block_barrier();
            }
        } else {
            for (int h = 0; h < nh; ++h) {
                __builtin_amdgcn_sched_barrier(0);
                load_frags(h);                           // phase 0: read half h
                __builtin_amdgcn_sched_barrier(0);
                mid_phase(h);
                mma();                                   // phase 1: compute half h
                __builtin_amdgcn_sched_barrier(0);
                block_barrier();
            }
        }

        // Values derived below are computed here, not hoisted above the K loop
        // (that would keep them live in registers across it).
        int opaque = 0;
        asm volatile("" : "+s"(opaque));
        const int c_row0 = row0 + opaque, c_row_end = row_end, c_col0 = col0 + opaque;
        mfma_drain();

        // ---- epilogue.  Lane holds token row (lane & 31) of each token fragment
        // and, for register v, weight-panel row (v/4)*8 + (lane/32)*4 + v%4.
        // Results go through a per-wave LDS staging area (the stage slots are
        // free now: 16 KiB per wave) so that global traffic is 16 bytes per lane
        // over whole row segments.
        uint16_t* stg = (wave < 4 ? s_a(0) : s_b(0)) + (wave & 3) * 8192 + opaque;
        const int wrow0 = c_row0 + GRP * WROWS;    // first token row of this wave
        if constexpr (EPI == EPI_STORE) {
            // [128 rows][64 cols] bf16 (128-byte rows); 8-byte unit u of row r at u ^ ((r >> 1) & 15)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r = i * 32 + (lane & 31);
                        const int u = j * 8 + q * 2 + (lane >> 5);
                        uint2 v;
                        v.x = pk(acc_rd(acc[i][j][q * 4 + 0]), acc_rd(acc[i][j][q * 4 + 1]));
                        v.y = pk(acc_rd(acc[i][j][q * 4 + 2]), acc_rd(acc[i][j][q * 4 + 3]));
                        *reinterpret_cast<uint2*>(stg + r * 64 + ((u ^ ((r >> 1) & 15)) << 2)) = v;
                    }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll 4
            for (int sidx = 0; sidx < 16; ++sidx) {
                const int idx = sidx * 64 + lane;
                const int r = idx >> 3, c = idx & 7;
                const int f = (r >> 1) & 15;
                uint4 v = *reinterpret_cast<const uint4*>(stg + r * 64 + ((c ^ (f >> 1)) << 3));
                if (f & 1) v = make_uint4(v.z, v.w, v.x, v.y);
                const int grow = wrow0 + r;
                const int gcol = c_col0 + wcol(c);
                if (grow < c_row_end && gcol < N)
                    *reinterpret_cast<uint4*>(p.out0 + static_cast<int64_t>(grow) * N + gcol) = v;
            }
        } else if constexpr (EPI == EPI_SWIGLU) {
            // two passes of 64 rows; per pass [64][32] bf16 arrays for A, gate, up
            // (64-byte rows); 8-byte unit u of row r at u ^ ((r >> 2) & 7)
            uint16_t* sA = stg;
            uint16_t* sG = stg + 2048;
            uint16_t* sU = stg + 4096;
#pragma unroll
            for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
                for (int ii = 0; ii < 2; ++ii) {
                    const int i = pass * 2 + ii;
                    const int prow = wrow0 + pass * 64 + ii * 32 + (lane & 31);
                    const float pr = (probs && prow < c_row_end) ? probs[prow] : 1.0f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r = ii * 32 + (lane & 31);
                        const int u = q * 2 + (lane >> 5);
                        const int off = r * 32 + ((u ^ ((r >> 2) & 7)) << 2);
                        swiglu4(acc[i][0], acc[i][1], q, slope, pr, probs != nullptr, *reinterpret_cast<uint2*>(sA + off),
                                *reinterpret_cast<uint2*>(sG + off), *reinterpret_cast<uint2*>(sU + off));
                    }
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int sidx = 0; sidx < 4; ++sidx) {
                    const int idx = sidx * 64 + lane;
                    const int r = idx >> 2, c = idx & 3;
                    const int f = (r >> 2) & 7;
                    const int off = r * 32 + ((c ^ (f >> 1)) << 3);
                    uint4 va = *reinterpret_cast<const uint4*>(sA + off);
                    uint4 vg = *reinterpret_cast<const uint4*>(sG + off);
                    uint4 vu = *reinterpret_cast<const uint4*>(sU + off);
                    if (f & 1) {
                        va = make_uint4(va.z, va.w, va.x, va.y);
                        vg = make_uint4(vg.z, vg.w, vg.x, vg.y);
                        vu = make_uint4(vu.z, vu.w, vu.x, vu.y);
                    }
                    const int grow = wrow0 + pass * 64 + r;
                    const int gcol = c_col0 + wq * 32 + c * 8;
                    if (grow < c_row_end && gcol < N) {
                        *reinterpret_cast<uint4*>(p.out0 + static_cast<int64_t>(grow) * N + gcol) = va;
                        if (p.out1) {
                            uint16_t* h = p.out1 + static_cast<int64_t>(grow) * (2 * N) + gcol;
                            *reinterpret_cast<uint4*>(h) = vg;
                            *reinterpret_cast<uint4*>(h + N) = vu;
                        }
                    }
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
        } else {
            // SwiGLU derivative.  Per pass of 64 rows the saved gate and up values
            // [64][64] each (128-byte rows) are copied into the staging area with
            // LDS-DMA; 16-byte chunk c of row r sits at c ^ ((r >> 1) & 7).  The
            // results overwrite them in place and leave as whole row segments.
            uint16_t* sG = stg;
            uint16_t* sU = stg + 4096;
            const uint32_t g_lds = lds_addr(sG), u_lds = lds_addr(sU);
#pragma unroll   // the accumulator index must stay compile-time
            for (int pass = 0; pass < 2; ++pass) {
                // copy: 64 rows x 128 bytes per array = 8 DMA instructions each
                const int prow0 = wrow0 + pass * 64;
                const uint16_t* hbase = p.aux + static_cast<int64_t>(uni(min(prow0, c_row_end - 1))) * (2 * N) +
                                        c_col0;
#pragma unroll
                for (int d = 0; d < 8; ++d) {
                    const int r = d * 8 + (lane >> 3);
                    const int c = (lane & 7) ^ ((r >> 1) & 7);
                    const int rr = min(prow0 + r, c_row_end - 1) - min(prow0, c_row_end - 1);
                    const int cc = min(c_col0 + wcol(c), N - 8) - c_col0;
                    const uint32_t voff = static_cast<uint32_t>((rr * 2 * N + cc) * 2);
                    dma16(hbase, voff, g_lds + d * 1024);
                    dma16(hbase + N, voff, u_lds + d * 1024);
                }
                wait_vmcnt<0>();
#pragma unroll
                for (int ii = 0; ii < 2; ++ii) {
                    const int i = pass * 2 + ii;
                    const int prow = prow0 + ii * 32 + (lane & 31);
                    const float pr = (probs && prow < c_row_end) ? probs[prow] : 1.0f;
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        // fragment j: output columns gc0 .. gc0 + 31
                        const int gc0 = c_col0 + j * (TBN / 2) + wq * 32;
                        float dps = 0.0f;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int r = ii * 32 + (lane & 31);
                            const int col = j * 32 + q * 8 + (lane >> 5) * 4;    // 4 columns
                            const bool cv = gc0 + q * 8 + (lane >> 5) * 4 < N;
                            const int off = r * 64 + (((col >> 3) ^ ((r >> 1) & 7)) << 3) + (col & 7);
                            const uint2 hg = *reinterpret_cast<const uint2*>(sG + off);
                            const uint2 hu = *reinterpret_cast<const uint2*>(sU + off);
                            const uint32_t gw[2] = {hg.x, hg.y};
                            const uint32_t uw[2] = {hu.x, hu.y};
                            const uint32_t dw[2] = {pk(acc_rd(acc[i][j][q * 4]), acc_rd(acc[i][j][q * 4 + 1])),
                                                    pk(acc_rd(acc[i][j][q * 4 + 2]), acc_rd(acc[i][j][q * 4 + 3]))};
                            float dg[4], du[4];
#pragma unroll
                            for (int x = 0; x < 4; ++x) {
                                const float g = (x & 1) ? hi_f(gw[x >> 1]) : lo_f(gw[x >> 1]);
                                const float u = (x & 1) ? hi_f(uw[x >> 1]) : lo_f(uw[x >> 1]);
                                const float da = (x & 1) ? hi_f(dw[x >> 1]) : lo_f(dw[x >> 1]);
                                const float sgm = __builtin_amdgcn_rcpf(1.0f + __expf(-(slope * g)));
                                const float dap = probs ? pr * da : da;
                                dg[x] = dap * u * sgm * (1.0f + slope * g * (1.0f - sgm));
                                du[x] = dap * g * sgm;
                                if (cv) dps += da * (g * sgm * u);
                            }
                            *reinterpret_cast<uint2*>(sG + off) =
                                make_uint2(pk(dg[0], dg[1]), pk(dg[2], dg[3]));
                            *reinterpret_cast<uint2*>(sU + off) =
                                make_uint2(pk(du[0], du[1]), pk(du[2], du[3]));
                        }
                        if (dp_part) {
                            // same per-lane order and halves as the streaming flavor
                            const float tot = dps + __shfl_xor(dps, 32, 64);
                            if (lane < 32 && prow < c_row_end && gc0 < N)
                                dp_part[static_cast<int64_t>(prow) * p.dp_ld + gc0 / 32] = tot;
                        }
                    }
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int sidx = 0; sidx < 8; ++sidx) {
                    const int idx = sidx * 64 + lane;
                    const int r = idx >> 3, c = idx & 7;
                    const int off = r * 64 + ((c ^ ((r >> 1) & 7)) << 3);
                    const uint4 vg = *reinterpret_cast<const uint4*>(sG + off);
                    const uint4 vu = *reinterpret_cast<const uint4*>(sU + off);
                    const int grow = prow0 + r;
                    const int gcol = c_col0 + wcol(c);
                    if (grow < c_row_end && gcol < N) {
                        uint16_t* dh = p.out0 + static_cast<int64_t>(grow) * (2 * N) + gcol;
                        *reinterpret_cast<uint4*>(dh) = vg;
                        *reinterpret_cast<uint4*>(dh + N) = vu;
                    }
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
        }
        };
        // Each group runs its own copy of the K loop and the epilogue, so its
        // accumulators never have to be merged with the other group's path.
        if (grp == 0) run_group(GrpTag<0>{}); else run_group(GrpTag<1>{});

        // every wave is done with the staging area before the next tile's copies
        block_barrier();
    }
}

// ---------------------------------------------------------------- four-wave kernel
//
// The four GEMMs over the caller's fragment-ordered copy of the weights (an
// optional buffer, for H % 256 == 0 and F % 128 == 0), each in one launch
// over a work list of thin items (the at most 96 rows an expert leaves after
// its 256-row tiles, or all rows of a small expert), then tiles; workgroups
// of even XCDs run their thin items first, those of odd XCDs their tiles
// first.  Four waves compute a 256 x 256 tile: wave w owns all 256 token
// rows and its own 64 weight rows (two 32-row blocks), as 8 x 2 accumulator
// blocks of 32 x 32 (all 256 AGPRs), so that no two waves load the same
// weight bytes.  Tokens stream
// through a 4-slot LDS ring of 64-k stages by LDS-DMA, three stages ahead,
// and each wave reads a step's eight token fragments from it.  Weights skip
// LDS: in the fragment-ordered copy the 64 lanes' 16-byte operands of one
// 32-row x 16-k block lie next to each other, so every lane loads its own
// MFMA operand straight into VGPRs with one coalesced 1 KiB load per block,
// seven k16 steps ahead into an 8-step register ring.  Every k16 step of a
// tile issues the same four loads (its two weight blocks seven steps ahead
// and two of the eight token copies of a stage three stages ahead; a thin
// item's step one copy of four), so the number of loads issued after any one
// of them is fixed and the waits are constant counts: a tile step's weights
// are complete at vmcnt(26) and a thin item's at vmcnt(19); a thin item's
// stage copies are complete at vmcnt(24), and in tiles the weight wait of a
// stage's last step already covers the next stage's copies.  Virtual steps
// before step 0 repeat the pattern as the prologue (without the weight loads
// that would come before the first real one, which no wait counts), and the
// steps past the end re-load clamped addresses, so the counts hold
// everywhere.  The sums are the same MFMA chain over k as in the eight-wave
// tiles and the streaming items, so a row's results do not depend on which
// flavor computed it.
//
// Fragment order: block b of 32 weight rows and k16 step s of an expert is
// 512 contiguous elements; lane l's 8 are rows 32b + (l & 31), k 16s + 8(l >> 5).
// For W1 the 32-row blocks go gate, gate, up, up per 64 features, so a wave's
// two blocks are the gate and up rows of the same 32 features.
constexpr int T4_THREADS = 256;
constexpr int T4_SLOT = 256 * BK;          // elements of one token stage
constexpr int T4_NSLOT = 4;

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Load one 16-byte weight fragment.  The register is an in/out operand so
// that a load's destination stays reserved until the next load into the same
// ring slot (also for the loads whose data is never used).
__device__ __forceinline__ void wfrag_load(bf16x8& w, const uint16_t* ptr) {
    asm volatile("global_load_dwordx4 %0, %1, off" : "+v"(w) : "v"(ptr) : "memory");
}
// The same load under a wave-uniform lane mask (all lanes, or lane 0 alone
// for a load whose data is not used): it is issued and counted like any
// other, but moves 16 bytes instead of 1 KiB.  The mask is set for this one
// instruction inside the asm block.
__device__ __forceinline__ void wfrag_load_m(bf16x8& w, const uint16_t* ptr, uint64_t mask) {
    uint64_t saved;
    asm volatile("s_mov_b64 %1, exec\n\t"
                 "s_mov_b64 exec, %3\n\t"
                 "global_load_dwordx4 %0, %2, off\n\t"
                 "s_mov_b64 exec, %1"
                 : "+v"(w), "=&s"(saved)
                 : "v"(ptr), "s"(mask)
                 : "memory");
}
#pragma clang diagnostic pop
// H1 = X W1^T over the fragment-ordered W1 (plain-store variant): the copy's
// 32-row block b holds W1 rows gate/up of 32 features (gate, gate, up, up per
// 64 features), so its outputs go to H1 column h1_col(b, F) onwards.
__device__ __forceinline__ int h1_col(int b, int F) {
    return ((b & 3) < 2 ? 0 : F) + (b >> 2) * 64 + (b & 1) * 32;
}
__device__ __forceinline__ int F_of(int N) { return N >> 1; }   // N = 2F for the H1 GEMM
// Waits for the weight fragments of the current step (at most N loads issued
// after them may be outstanding) tie the registers they guard, so that nothing
// reads them before the wait.  A thin item's step: two weight blocks, 19
// later loads.
__device__ __forceinline__ void wfrag_wait19(bf16x8& a, bf16x8& b) {
    asm volatile("s_waitcnt vmcnt(19)" : "+v"(a), "+v"(b) :: "memory");
}
// Ties two registers without a wait (after a wait that covers them).
__device__ __forceinline__ void wfrag_hold2(bf16x8& a, bf16x8& b) {
    asm volatile("" : "+v"(a), "+v"(b) :: "memory");
}
// A tile's step: its two weight blocks are complete at vmcnt(26) (the same
// step's two token copies plus six steps of two loads and two copies after them).
__device__ __forceinline__ void wfrag_wait26(bf16x8& a, bf16x8& b) {
    asm volatile("s_waitcnt vmcnt(26)" : "+v"(a), "+v"(b) :: "memory");
}

// The activation derivative of four consecutive features of one token row,
// in place: g, u are the saved bf16 gate and up values at pg and pu, the
// results dG, dU overwrite them; dA = bf16(a[4q + x]).  The same arithmetic,
// in the same order, as the eight-wave kernel's derivative epilogues: plain
// SwiGLU without EXT; with EXT the sigmoid slope, the row's probability pr
// (when weighted) and the row's dp partial sum dps, which gains the four
// features' da * act(g) * u in increasing x.
template <bool EXT>
__device__ __forceinline__ void dswiglu_inplace(uint16_t* pg, uint16_t* pu, const f32x16& a, int q, float slope,
                                                float pr, bool weighted, float& dps) {
    const uint2 hg = *reinterpret_cast<const uint2*>(pg);
    const uint2 hu = *reinterpret_cast<const uint2*>(pu);
    const uint32_t gw[2] = {hg.x, hg.y};
    const uint32_t uw[2] = {hu.x, hu.y};
    const uint32_t dw[2] = {pack2(acc_rd(a[q * 4]), acc_rd(a[q * 4 + 1])), pack2(acc_rd(a[q * 4 + 2]), acc_rd(a[q * 4 + 3]))};
    float dg[4], du[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const float g = (x & 1) ? hi_f(gw[x >> 1]) : lo_f(gw[x >> 1]);
        const float u = (x & 1) ? hi_f(uw[x >> 1]) : lo_f(uw[x >> 1]);
        const float da = (x & 1) ? hi_f(dw[x >> 1]) : lo_f(dw[x >> 1]);
        if constexpr (EXT) {
            const float sgm = __builtin_amdgcn_rcpf(1.0f + __expf(-(slope * g)));
            const float dap = weighted ? pr * da : da;
            dg[x] = dap * u * sgm * (1.0f + slope * g * (1.0f - sgm));
            du[x] = dap * g * sgm;
            dps += da * (g * sgm * u);
        } else {
            const float sgm = __builtin_amdgcn_rcpf(1.0f + __expf(-(1.0f * g)));
            dg[x] = da * u * sgm * (1.0f + 1.0f * g * (1.0f - sgm));
            du[x] = da * g * sgm;
        }
    }
    *reinterpret_cast<uint2*>(pg) = make_uint2(pack2(dg[0], dg[1]), pack2(dg[2], dg[3]));
    *reinterpret_cast<uint2*>(pu) = make_uint2(pack2(du[0], du[1]), pack2(du[2], du[3]));
}

template <int EPI, bool EXT>
__global__ __launch_bounds__(T4_THREADS, 1)
void tile4_kernel(const GemmParams p) {
    static_assert(EPI == EPI_STORE || EPI == EPI_SWIGLU || EPI == EPI_DSWIGLU,
                  "store, SwiGLU and the activation derivative");
    const float slope = EXT ? p.slope : 1.0f;
    const float* const probs = EXT ? p.probs : nullptr;
    __shared__ __attribute__((aligned(1024))) uint16_t s_ring[T4_NSLOT * T4_SLOT];
    __shared__ int s_off[GG_KMAX_EXPERTS + 1];
    __shared__ int s_pre[GG_KMAX_EXPERTS + 1];
    __shared__ int s_spre[GG_KMAX_EXPERTS + 1];
    const int E = p.E, M = p.M, K = p.K, N = p.N;
    constexpr int TILE_COLS = (EPI == EPI_SWIGLU) ? TBN / 2 : TBN;
    const int tiles_n = N / TILE_COLS;
    // thin items (the at most 96 rows an expert leaves after its tiles) use
    // the tiles' column blocks
    build_schedule<T4_THREADS>(p.offsets, E, M, tiles_n, tiles_n, s_off, s_pre, s_spre);
    const int n_items = uni(s_spre[E]);
    const int n_tiles = uni(s_pre[E]);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = uni(tid >> 6);
    const int kiters = K / BK, nsteps = K / 16;
    const int G = gridDim.x, b = blockIdx.x;
    const int slot = (G % 8 == 0) ? (b & 7) * (G >> 3) + (b >> 3) : b;
    const uint32_t ring_l = lds_addr(s_ring);
    // LDS-DMA: lane tid moves chunk (tid & 7) of row (tid >> 3) + 32 i; the
    // logical k chunk stored there follows the [row][64 k] swizzle.
    const int lc = ((tid & 7) ^ kswz(tid >> 3)) * 8;

    f32x16 acc[8][2];
    bf16x8 wr[8][2];
    bf16x8 tf[2][8];

    // ---- thin items: rows x TILE_COLS output columns.  Each wave owns
    // two 32-row weight blocks (for SwiGLU the gate and up rows of 32
    // features) against three 32-row token blocks.  Per k16 step: two weight
    // loads seven steps ahead and one of the four token copies of the stage
    // three stages ahead (128 rows, the ones past the item clamped), so a
    // step's weights are complete at vmcnt(19) and a stage's tokens at
    // vmcnt(24).
    //   A thin item is bound by the bytes its workgroup moves.  When the
    // thin items fit into the grid twice over, each is split into two halves
    // of its columns, so twice as many workgroups share its weight bytes.
    // A half keeps the loop as it is: for plain stores each wave owns one
    // 32-row block (its second load and MFMAs repeat the first); for SwiGLU
    // waves 0 and 1 own the gate and up blocks of the half's 32 + 32
    // features and waves 2 and 3 repeat them.  The repeated loads run on one
    // lane, the repeated results are not stored, and a row's arithmetic is
    // the same either way.
    constexpr bool THIN_HALVES = EPI != EPI_DSWIGLU;
    const int h_sh = (THIN_HALVES && 2 * n_items <= G) ? 1 : 0;   // log2 of the work units per thin item
    const int n_units = n_items << h_sh;
    // Workgroup s takes units s, s + G, ... of the work list (thin units,
    // then tiles).  The workgroups of every other XCD (blockIdx mod 8) run
    // their tiles before their thin units, so that half of the chip reaches
    // the tile boundaries (the epilogue stores and the next tile's first
    // loads) at other times than the other half, while the workgroups of one
    // XCD, which share operand panels in its L2, stay in step.
    const bool tiles_first = (b & 1) != 0;
    int t_first = slot;
    if (t_first < n_units) t_first += (n_units - t_first + G - 1) / G * G;
    t_first -= n_units;
    for (int phase = 0; phase < 2; ++phase) {
        const bool thin_now = (phase == 0) != tiles_first;
        for (int wi = thin_now ? slot : n_units; wi < n_units; wi += G) {
            const int ti = wi >> h_sh;     // thin item
            const int hf = wi & h_sh;      // its half (0 for a whole item)
            const int e = uni(find_expert(s_spre, E, ti));
            const int local = ti - uni(s_spre[e]);
            const int rb = uni(s_off[e]);
            const int re = uni(s_off[e + 1]);
            const int row0 = uni(rb + tile_rows_of(re - rb));
            const int rows = re - row0;                          // 1 .. 96
            const int col0 = uni(local * TILE_COLS);
            const uint16_t* a_base = p.act + static_cast<int64_t>(row0) * K;
            const uint16_t* wfe = p.wfrag + static_cast<int64_t>(e) * p.wfrag_stride;
            const int tb0 = (EPI == EPI_SWIGLU) ? (col0 / 64 + (h_sh ? hf : (wave >> 1))) * 4 + (wave & 1)
                                                : col0 / 32 + (h_sh ? 4 * hf + wave : 2 * wave);
            const int tb1 = (EPI == EPI_SWIGLU) ? tb0 + 2 : (h_sh ? tb0 : tb0 + 1);
            // loads whose results a half item does not store move one lane only
            const bool rep0 = h_sh && EPI == EPI_SWIGLU && wave >= 2;
            const bool rep1 = h_sh && (EPI != EPI_SWIGLU || wave >= 2);
            const uint64_t lm0 = uni(rep0) ? 1ull : ~0ull;
            const uint64_t lm1 = uni(rep1) ? 1ull : ~0ull;
            auto wp = [&](int g, int j) -> const uint16_t* {
                return wfe + ((static_cast<int64_t>(j ? tb1 : tb0) * nsteps + g) * 64 + lane) * 8;
            };
            auto tdma1 = [&](int s, int part) {
                const int ss = s < kiters ? s : kiters - 1;
                const int r = min((tid >> 3) + 32 * part, rows - 1);
                const uint32_t lds = ring_l + (s & 3) * (T4_SLOT * 2) + (wave * 64 + T4_THREADS * part) * 16;
                dma16(a_base, static_cast<uint32_t>((r * K + ss * BK + lc) * 2), lds);
            };
            auto rd3 = [&](int g, int buf) {
                const uint16_t* st = s_ring + ((g >> 2) & 3) * T4_SLOT;
                const int ch = 2 * (g & 3) + (lane >> 5);
#pragma unroll
                for (int i = 0; i < 3; ++i)
                    tf[buf][i] = *reinterpret_cast<const bf16x8*>(st + kc_off(i * 32 + (lane & 31), ch));
            };
            // prologue: virtual steps -12..-1; steps -12..-8 issue no weight loads
            // (they come before the first one, so no weight wait counts them).
            // Stage 0's last copy is then followed by 22 loads, not the 24 the
            // loop's stage wait assumes, so the prologue waits for it here.
#pragma unroll
            for (int g = -12; g < 0; ++g) {
                const int gw = g + 7;
                if (gw >= 0) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) wfrag_load_m(wr[gw & 7][j], wp(gw, j), j ? lm1 : lm0);
                }
                tdma1((g >> 2) + 3, g & 3);
            }
            wait_vmcnt<22>();
            // K step g (u = g % 8).  The item's first step starts its sums from
            // an immediate zero, so the accumulators are never cleared.
            auto kstep = [&](int g, auto u_tag, auto first_tag) {
                constexpr int u = decltype(u_tag)::value;
                constexpr int j4 = u & 3;
                if constexpr (j4 == 0) {
                    wait_vmcnt<24>();
                    block_barrier();
                    rd3(g, u & 1);
                }
                if constexpr (j4 < 3) rd3(g + 1, (u + 1) & 1);
                wfrag_wait19(wr[u][0], wr[u][1]);
#pragma unroll
                for (int i = 0; i < 3; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        if constexpr (decltype(first_tag)::value != 0)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wr[u][j], tf[u & 1][i], f32x16{}, 0, 0, 0);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wr[u][j], tf[u & 1][i], acc[i][j], 0, 0, 0);
                    }
                const int gw = g + 7;
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    wfrag_load_m(wr[(u + 7) & 7][j], wp(gw < nsteps ? gw : nsteps - 1, j), j ? lm1 : lm0);
                tdma1((g >> 2) + 3, j4);
            };
            static_for<8>([&](auto ut) { kstep(decltype(ut)::value, ut, GrpTag<(decltype(ut)::value == 0)>{}); });
            for (int g0 = 8; g0 < nsteps; g0 += 8)
                static_for<8>([&](auto ut) { kstep(g0 + decltype(ut)::value, ut, GrpTag<0>{}); });
            wait_vmcnt<0>();
#pragma unroll
            for (int s = 0; s < 8; ++s) wfrag_hold2(wr[s][0], wr[s][1]);
            block_barrier();
            mfma_drain();
            int opaque = 0;
            asm volatile("" : "+s"(opaque));
            const int trow0 = row0 + opaque;
            uint16_t* stg = s_ring + wave * T4_SLOT + opaque;   // 32 KiB per wave
            if constexpr (EPI == EPI_STORE) {
                // [96 rows][64 cols] bf16; 16-byte chunk c of row r at c ^ (r & 7)
#pragma unroll
                for (int i = 0; i < 3; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int r = i * 32 + (lane & 31);
                            const int c = j * 4 + q;
                            uint2 v;
                            v.x = pack2(acc_rd(acc[i][j][q * 4 + 0]), acc_rd(acc[i][j][q * 4 + 1]));
                            v.y = pack2(acc_rd(acc[i][j][q * 4 + 2]), acc_rd(acc[i][j][q * 4 + 3]));
                            *reinterpret_cast<uint2*>(stg + r * 64 + ((c ^ (r & 7)) << 3) + 4 * (lane >> 5)) = v;
                        }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                // a half item's wave stores its first 32 columns (block tb0) only
                const int gcol0 = col0 + (h_sh ? 128 * hf + 32 * wave : 64 * wave);
#pragma unroll 4
                for (int sidx = 0; sidx < 12; ++sidx) {
                    const int idx = sidx * 64 + lane;
                    const int r = idx >> 3, c = idx & 7;
                    const uint4 v = *reinterpret_cast<const uint4*>(stg + r * 64 + ((c ^ (r & 7)) << 3));
                    const int oc = p.h1_order ? h1_col(tb0 + (c >> 2), F_of(N)) + (c & 3) * 8 : gcol0 + c * 8;
                    if (r < rows && (!h_sh || c < 4))
                        *reinterpret_cast<uint4*>(p.out0 + static_cast<int64_t>(trow0 + r) * N + oc) = v;
                }
            } else if constexpr (EPI == EPI_DSWIGLU) {
                // The saved gate and up values of the wave's 64 features for the
                // item's rows, [96 rows][gate 64 | up 64] bf16 (256-byte rows,
                // 24 KiB), are copied into the staging area with LDS-DMA (rows past
                // the item repeat its last row); 16-byte chunk c (0..7 gate, 8..15
                // up) of row r sits at (c & 8) | ((c & 7) ^ (r & 7)).  The results
                // overwrite them in place and leave as whole row segments of dH1.
                const int F = N;
                const int f0 = col0 + 64 * wave + opaque;
                const int ln = lane + opaque;     // per-lane values computed here, not above the K loop
                const uint16_t* hb = p.aux + static_cast<int64_t>(row0) * (2 * F);
                const uint32_t sl = lds_addr(stg);
#pragma unroll
                for (int d = 0; d < 24; ++d) {
                    const int r = 4 * d + (ln >> 4), pc = ln & 15;
                    const int c = (pc & 8) | ((pc & 7) ^ (r & 7));
                    const int col = (c < 8 ? 0 : F) + f0 + 8 * (c & 7);
                    dma16(hb, static_cast<uint32_t>((min(r, rows - 1) * 2 * F + col) * 2), sl + d * 1024);
                }
                wait_vmcnt<0>();
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    const int r = i * 32 + (ln & 31);
                    const float pr = (probs && r < rows) ? probs[trow0 + r] : 1.0f;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        float dps = 0.0f;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int pos = (4 * j + q) ^ (r & 7);
                            uint16_t* pg = stg + r * 128 + pos * 8 + 4 * (ln >> 5);
                            dswiglu_inplace<EXT>(pg, pg + 64, acc[i][j], q, slope, pr, probs != nullptr, dps);
                        }
                        if (EXT && p.dp_part) {
                            // the 32 features' partial sum, in the eight-wave kernel's order
                            const float tot = dps + __shfl_xor(dps, 32, 64);
                            if (ln < 32 && r < rows)
                                p.dp_part[static_cast<int64_t>(trow0 + r) * p.dp_ld + (f0 + 32 * j) / 32] = tot;
                        }
                    }
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll 4
                for (int d = 0; d < 24; ++d) {
                    const int r = 4 * d + (ln >> 4), pc = ln & 15;
                    const int c = (pc & 8) | ((pc & 7) ^ (r & 7));
                    const uint4 v = *reinterpret_cast<const uint4*>(stg + r * 128 + pc * 8);
                    const int col = (c < 8 ? 0 : F) + f0 + 8 * (c & 7);
                    if (r < rows) *reinterpret_cast<uint4*>(p.out0 + static_cast<int64_t>(trow0 + r) * (2 * F) + col) = v;
                }
            } else {
                // [96 rows][32 features] bf16 arrays for A, gate and up; 16-byte
                // chunk c of row r at c ^ (r & 3)
                uint16_t* sA = stg;
                uint16_t* sG = stg + 3072;
                uint16_t* sU = stg + 6144;
                // a half item's features are stored by waves 0 and 1
                const int fcol0 = col0 + (h_sh ? 64 * hf : 0) + 32 * wave;
                const bool owns = !h_sh || wave < 2;
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    const int r = i * 32 + (lane & 31);
                    const float pr = (probs && r < rows) ? probs[trow0 + r] : 1.0f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int off = r * 32 + ((q ^ (r & 3)) << 3) + 4 * (lane >> 5);
                        swiglu4(acc[i][0], acc[i][1], q, slope, pr, probs != nullptr, *reinterpret_cast<uint2*>(sA + off),
                                *reinterpret_cast<uint2*>(sG + off), *reinterpret_cast<uint2*>(sU + off));
                    }
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll 2
                for (int sidx = 0; sidx < 6; ++sidx) {
                    const int idx = sidx * 64 + lane;
                    const int r = idx >> 2, c = idx & 3;
                    const int off = r * 32 + ((c ^ (r & 3)) << 3);
                    const uint4 va = *reinterpret_cast<const uint4*>(sA + off);
                    const uint4 vg = *reinterpret_cast<const uint4*>(sG + off);
                    const uint4 vu = *reinterpret_cast<const uint4*>(sU + off);
                    if (r < rows && owns) {
                        *reinterpret_cast<uint4*>(p.out0 + static_cast<int64_t>(trow0 + r) * N + fcol0 + c * 8) = va;
                        if (p.out1) {
                            uint16_t* h = p.out1 + static_cast<int64_t>(trow0 + r) * (2 * N) + fcol0 + c * 8;
                            *reinterpret_cast<uint4*>(h) = vg;
                            *reinterpret_cast<uint4*>(h + N) = vu;
                        }
                    }
                }
            }
            block_barrier();   // staging reads done before the next copies land
        }

        // ---- the 256-row tiles.  Wave w owns all 256 token rows and its own
        // 64 weight rows (two 32-row blocks: for SwiGLU the gate and up rows of 32
        // features, else 64 output columns), as 8 x 2 accumulator blocks of
        // 32 x 32 (all 256 AGPRs).  So no two waves load the same weight bytes:
        // per k16 step a workgroup moves 8 KiB of weights and 8 KiB of token
        // copies through the vector-memory path, and each wave reads the step's
        // eight token fragments from the LDS ring, one step ahead.  Per k16 step
        // every wave issues two weight loads (seven steps ahead) and two of the
        // eight token copies of a stage three stages ahead: stage s + 4 in steps
        // 4s + 3 .. 4s + 6, after the barrier of step 4s + 3 (the last of stage s)
        // has freed slot s % 4.  A step's weights are complete at vmcnt(26)
        // (2 + 6 x 4), and that wait in step 4s + 3 also covers this wave's
        // copies of stage s + 1, the last of which has 28 loads after it; so the
        // barrier there lets every wave read the first fragments of stage s + 1
        // a step ahead like all others.
        for (int t = thin_now ? n_tiles : t_first; t < n_tiles; t += G) {
            const int e = uni(find_expert(s_pre, E, t));
            const int local = t - uni(s_pre[e]);
            const int rb = uni(s_off[e]);
            const int row_end = uni(s_off[e + 1]);
            const int tiles_m = tiles_m_of(row_end - rb);
            const int row0 = uni(rb + (local % tiles_m) * TBM);
            const int col0 = uni((local / tiles_m) * TILE_COLS);
            const int rows = min(TBM, row_end - row0);
            const uint16_t* a_base = p.act + static_cast<int64_t>(row0) * K;
            const uint16_t* wfe = p.wfrag + static_cast<int64_t>(e) * p.wfrag_stride;
            // this wave's two 32-row blocks in fragment order (W1's blocks go gate,
            // gate, up, up per 64 features)
            const int wb0 = (EPI == EPI_SWIGLU) ? (col0 / 64 + (wave >> 1)) * 4 + (wave & 1) : col0 / 32 + 2 * wave;
            const int wb1 = (EPI == EPI_SWIGLU) ? wb0 + 2 : wb0 + 1;
            auto wptr = [&](int g, int j) -> const uint16_t* {
                return wfe + ((static_cast<int64_t>(j ? wb1 : wb0) * nsteps + g) * 64 + lane) * 8;
            };
            // two of the eight LDS-DMA instructions of token stage s (clamped to the last)
            auto tdma = [&](int s, int part) {
                const int ss = s < kiters ? s : kiters - 1;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int i = 2 * part + u;
                    const int r = min((tid >> 3) + 32 * i, rows - 1);
                    const uint32_t lds = ring_l + (s & 3) * (T4_SLOT * 2) + (wave * 64 + T4_THREADS * i) * 16;
                    dma16(a_base, static_cast<uint32_t>((r * K + ss * BK + lc) * 2), lds);
                }
            };
            auto rd_t = [&](int g, int buf) {   // the eight token fragments of step g
                const uint16_t* st = s_ring + ((g >> 2) & 3) * T4_SLOT;
                const int ch = 2 * (g & 3) + (lane >> 5);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    tf[buf][i] = *reinterpret_cast<const bf16x8*>(st + kc_off(i * 32 + (lane & 31), ch));
            };
            // prologue: virtual steps -13..-1 (weights of steps 0..6 from step -7
            // on, token stages 0..2 and the first copy of stage 3); step -1 ends
            // like the last step of a stage: stage 0 is in, and its first step's
            // fragments are read.  Steps -13..-8 issue no weight loads: they come
            // before the first one, so no weight wait counts them, and 28 loads
            // follow stage 0's last copy (steps -9 and -8 issue two, -7..-2 four).
#pragma unroll
            for (int g = -13; g < 0; ++g) {
                const int gw = g + 7;
                if (g == -1) {
                    wait_vmcnt<28>();    // this wave's copies of stage 0
                    block_barrier();
                    rd_t(0, 0);
                }
                if (gw >= 0) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) wfrag_load(wr[gw & 7][j], wptr(gw, j));
                }
                tdma(((g + 1) >> 2) + 3, (g + 1) & 3);
            }
            // K step g (u = g % 8).  The tile's first step starts its sums from
            // an immediate zero, so the accumulators are never cleared.
            auto kstep = [&](int g, auto u_tag, auto first_tag) {
                constexpr int u = decltype(u_tag)::value;
                constexpr int j4 = u & 3;
                // this step's weights; in a stage's last step also this wave's
                // copies of the next stage (28 loads were issued after them)
                wfrag_wait26(wr[u][0], wr[u][1]);
                // In a stage's last step: every wave's copies of the next
                // stage are in, and every wave has read all of this stage's
                // fragments, so its slot may be refilled from here on.
                if constexpr (j4 == 3) block_barrier();
                rd_t(g + 1, (u + 1) & 1);
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        if constexpr (decltype(first_tag)::value != 0)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wr[u][j], tf[u & 1][i], f32x16{}, 0, 0, 0);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wr[u][j], tf[u & 1][i], acc[i][j], 0, 0, 0);
                    }
                const int gw = g + 7;
#pragma unroll
                for (int j = 0; j < 2; ++j) wfrag_load(wr[(u + 7) & 7][j], wptr(gw < nsteps ? gw : nsteps - 1, j));
                tdma(((g + 1) >> 2) + 3, (j4 + 1) & 3);
                // issue order within the step: one token fragment read for the
                // next step after each of the first eight MFMAs, so the reads
                // spread over the step instead of bunching behind its MFMAs
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            };
            static_for<8>([&](auto ut) { kstep(decltype(ut)::value, ut, GrpTag<(decltype(ut)::value == 0)>{}); });
            for (int g0 = 8; g0 < nsteps; g0 += 8)
                static_for<8>([&](auto ut) { kstep(g0 + decltype(ut)::value, ut, GrpTag<0>{}); });
            // drain the clamped loads; the ring becomes the epilogue's staging area
            wait_vmcnt<0>();
#pragma unroll
            for (int s = 0; s < 8; ++s) wfrag_hold2(wr[s][0], wr[s][1]);
            block_barrier();
            mfma_drain();
            // Values derived below are computed here, not hoisted above the K loop.
            int opaque = 0;
            asm volatile("" : "+s"(opaque));
            const int trow0 = row0 + opaque;
            const int ln = lane + opaque;
            uint16_t* stg = s_ring + wave * T4_SLOT + opaque;   // 32 KiB per wave
            // Lane holds token row (ln & 31) of each token block i and, for
            // register 4q + x of block j, weight row 32j + 8q + 4(ln >> 5) + x of
            // the wave's 64.
            if constexpr (EPI == EPI_STORE) {
                // [256 rows][64 cols] bf16 (128-byte rows); 16-byte chunk c of row r at c ^ (r & 7)
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int r = i * 32 + (ln & 31);
                            const int c = j * 4 + q;
                            uint2 v;
                            v.x = pack2(acc_rd(acc[i][j][q * 4 + 0]), acc_rd(acc[i][j][q * 4 + 1]));
                            v.y = pack2(acc_rd(acc[i][j][q * 4 + 2]), acc_rd(acc[i][j][q * 4 + 3]));
                            *reinterpret_cast<uint2*>(stg + r * 64 + ((c ^ (r & 7)) << 3) + 4 * (ln >> 5)) = v;
                        }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                const int gcol0 = col0 + 64 * wave;
#pragma unroll 4
                for (int sidx = 0; sidx < 32; ++sidx) {
                    const int idx = sidx * 64 + ln;
                    const int r = idx >> 3, pc = idx & 7;
                    const int c = pc ^ (r & 7);
                    const uint4 v = *reinterpret_cast<const uint4*>(stg + r * 64 + pc * 8);
                    const int oc = p.h1_order ? h1_col(wb0 + (c >> 2), F_of(N)) + (c & 3) * 8 : gcol0 + c * 8;
                    if (r < rows) *reinterpret_cast<uint4*>(p.out0 + static_cast<int64_t>(trow0 + r) * N + oc) = v;
                }
            } else if constexpr (EPI == EPI_SWIGLU) {
                // two passes of 128 token rows; per pass [128][32] bf16 arrays for
                // A, gate and up (64-byte rows); 16-byte chunk c of row r at c ^ (r & 3)
                uint16_t* sA = stg;
                uint16_t* sG = stg + 4096;
                uint16_t* sU = stg + 8192;
                const int fcol0 = col0 + 32 * wave;        // first feature of this wave
#pragma unroll
                for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        const int i = pass * 4 + ii;
                        const int r = ii * 32 + (ln & 31);
                        const int prow = trow0 + pass * 128 + r;
                        const float pr = (probs && prow < row_end) ? probs[prow] : 1.0f;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int off = r * 32 + ((q ^ (r & 3)) << 3) + 4 * (ln >> 5);
                            swiglu4(acc[i][0], acc[i][1], q, slope, pr, probs != nullptr,
                                    *reinterpret_cast<uint2*>(sA + off), *reinterpret_cast<uint2*>(sG + off),
                                    *reinterpret_cast<uint2*>(sU + off));
                        }
                    }
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll 2
                    for (int sidx = 0; sidx < 8; ++sidx) {
                        const int idx = sidx * 64 + ln;
                        const int r = idx >> 2, pc = idx & 3;
                        const int c = pc ^ (r & 3);
                        const int off = r * 32 + pc * 8;
                        const int grow = trow0 + pass * 128 + r;
                        const uint4 va = *reinterpret_cast<const uint4*>(sA + off);
                        const uint4 vg = *reinterpret_cast<const uint4*>(sG + off);
                        const uint4 vu = *reinterpret_cast<const uint4*>(sU + off);
                        if (grow < row_end) {
                            *reinterpret_cast<uint4*>(p.out0 + static_cast<int64_t>(grow) * N + fcol0 + c * 8) = va;
                            if (p.out1) {
                                uint16_t* h = p.out1 + static_cast<int64_t>(grow) * (2 * N) + fcol0 + c * 8;
                                *reinterpret_cast<uint4*>(h) = vg;
                                *reinterpret_cast<uint4*>(h + N) = vu;
                            }
                        }
                    }
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                }
            } else {
                // SwiGLU derivative.  Per pass of 64 token rows (token blocks 2p,
                // 2p + 1) the saved gate and up values of the wave's 64 features,
                // [64 rows][gate 64 | up 64] bf16 (256-byte rows, 16 KiB), are
                // copied into one of two staging buffers with LDS-DMA (rows past
                // the tile repeat its last row); 16-byte chunk c (0..7 gate, 8..15
                // up) of row r sits at (c & 8) | ((c & 7) ^ (r & 7)).  The next
                // pass's copy is in flight while a pass is computed in place and
                // stored as whole row segments of dH1.  The waits count this wave's
                // memory operations in issue order: 16 copies or 16 stores a pass.
                const int F = N;
                const int f0 = col0 + 64 * wave + opaque;
                const int trows = rows + opaque;
                const uint16_t* hb = p.aux + static_cast<int64_t>(row0) * (2 * F);
                const uint32_t sl = lds_addr(stg);
                auto h1_copy = [&](int pass, int buf) {
#pragma unroll
                    for (int d = 0; d < 16; ++d) {
                        const int r = 4 * d + (ln >> 4), pc = ln & 15;
                        const int c = (pc & 8) | ((pc & 7) ^ (r & 7));
                        const int trow = min(pass * 64 + r, trows - 1);
                        const int col = (c < 8 ? 0 : F) + f0 + 8 * (c & 7);
                        dma16(hb, static_cast<uint32_t>((trow * 2 * F + col) * 2), sl + buf * 16384 + d * 1024);
                    }
                };
                auto h1_compute = [&](auto pass_tag, int buf) {
                    constexpr int pass = decltype(pass_tag)::value;
                    uint16_t* bb = stg + buf * 8192;
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) {
                        const int r = ii * 32 + (ln & 31);
                        const int prow = trow0 + pass * 64 + r;
                        const float pr = (probs && prow < row_end) ? probs[prow] : 1.0f;
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            float dps = 0.0f;
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const int pos = (4 * j + q) ^ (r & 7);
                                uint16_t* pg = bb + r * 128 + pos * 8 + 4 * (ln >> 5);
                                dswiglu_inplace<EXT>(pg, pg + 64, acc[2 * pass + ii][j], q, slope, pr,
                                                     probs != nullptr, dps);
                            }
                            if (EXT && p.dp_part) {
                                // the 32 features' partial sum, in the eight-wave kernel's order
                                const float tot = dps + __shfl_xor(dps, 32, 64);
                                if (ln < 32 && prow < row_end)
                                    p.dp_part[static_cast<int64_t>(prow) * p.dp_ld + (f0 + 32 * j) / 32] = tot;
                            }
                        }
                    }
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                };
                auto h1_store = [&](int pass, int buf) {
                    const uint16_t* bb = stg + buf * 8192;
#pragma unroll
                    for (int d = 0; d < 16; ++d) {
                        const int r = 4 * d + (ln >> 4), pc = ln & 15;
                        const int c = (pc & 8) | ((pc & 7) ^ (r & 7));
                        const uint4 v = *reinterpret_cast<const uint4*>(bb + r * 128 + pc * 8);
                        const int grow = trow0 + pass * 64 + r;
                        const int col = (c < 8 ? 0 : F) + f0 + 8 * (c & 7);
                        if (grow < row_end)
                            *reinterpret_cast<uint4*>(p.out0 + static_cast<int64_t>(grow) * (2 * F) + col) = v;
                    }
                    // the buffer's reads are done before a copy refills it
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                };
                // The compiler skips a store instruction whose 64 lanes all lie
                // past the tile, so the counts that include stores hold only
                // where all of them are issued: pass 0 always (a tile has more
                // than 96 rows), passes 1 and 2 in full tiles.  A partial tile
                // waits for every store before the copy it needs instead, so no
                // copy of it is still in flight when the next tile's copies land.
                const bool full = rows == TBM;
                h1_copy(0, 0);
                h1_copy(1, 1);
                wait_vmcnt<16>();                       // pass 0 has landed
                h1_compute(GrpTag<0>{}, 0);
                h1_store(0, 0);
                h1_copy(2, 0);
                wait_vmcnt<32>();                       // pass 1 (then the stores of pass 0, the copy of pass 2)
                h1_compute(GrpTag<1>{}, 1);
                h1_store(1, 1);
                h1_copy(3, 1);
                if (full) wait_vmcnt<32>();             // pass 2 (then the stores of pass 1, the copy of pass 3)
                else wait_vmcnt<16>();
                h1_compute(GrpTag<2>{}, 0);
                h1_store(2, 0);
                if (full) wait_vmcnt<16>();             // pass 3 (then the stores of pass 2)
                else wait_vmcnt<0>();
                h1_compute(GrpTag<3>{}, 1);
                h1_store(3, 1);
            }
            block_barrier();   // staging reads done before the next tile's copies land
        }
    }
}


// Fragment-ordered copies (layout above) of every expert's W1 and W2 for the
// forward tiles, of W1^T [H][2F] for dX = dH1 W1 and of W2^T [F][H] for
// dA = dY W2, written into the caller's fragment buffer (expert blocks of
// FRAG_BLOCK_FH * F * H elements: W1 at FRAG_W1, W2 at FRAG_W2, W1^T at
// FRAG_W1T, W2^T at FRAG_W2T, in units of F * H) from the row-major matrices
// of the packed buffer (expert blocks of 3 * F * H).
__global__ void pack_frag_kernel(const uint16_t* __restrict__ packed, uint16_t* __restrict__ frag, int E, int H,
                                 int F) {
    const int64_t fh = static_cast<int64_t>(F) * H;
    // One thread per 16-byte chunk of the fragment buffer.  A chunk's matrix
    // follows from its element offset inside its expert block, so the writes
    // cover exactly E * FRAG_BLOCK_FH * F * H elements.
    const int64_t per_e = FRAG_BLOCK_FH * fh / 8;
    const int64_t total = static_cast<int64_t>(E) * per_e;
    const int64_t step = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += step) {
        const int e = static_cast<int>(i / per_e);
        const int64_t el = (i - static_cast<int64_t>(e) * per_e) * 8;    // element offset in the block
        const int at = el < FRAG_W2 * fh ? FRAG_W1 : (el < FRAG_W1T * fh ? FRAG_W2 : (el < FRAG_W2T * fh ? FRAG_W1T : FRAG_W2T));
        const int64_t ci = (el - at * fh) / 8;                           // chunk within its matrix
        const uint16_t* blk = packed + e * 3 * fh;                       // row-major W1_e, then W2_e
        const int K = at == FRAG_W1 ? H : (at == FRAG_W2 ? F : (at == FRAG_W1T ? 2 * F : H));
        const int l = static_cast<int>(ci & 63);
        const int64_t rest = ci >> 6;
        const int ks = static_cast<int>(rest % (K / 16));
        const int rbk = static_cast<int>(rest / (K / 16));
        const int k0 = ks * 16 + (l >> 5) * 8;
        uint16_t* dst = frag + e * FRAG_BLOCK_FH * fh + el;
        const int row = rbk * 32 + (l & 31);
        if (at == FRAG_W1T || at == FRAG_W2T) {   // row n of the transpose is column n of the matrix
            const uint16_t* src = at == FRAG_W1T ? blk : blk + 2 * fh;   // W1 [2F][H] or W2 [H][F]
            const int ld = at == FRAG_W1T ? H : F;
            uint16_t v[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) v[x] = src[static_cast<int64_t>(k0 + x) * ld + row];
            *reinterpret_cast<uint4*>(dst) = make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16),
                                                        v[4] | (v[5] << 16), v[6] | (v[7] << 16));
            continue;
        }
        int srow = row;
        if (at == FRAG_W1) {
            const int q = rbk & 3, fb = rbk >> 2;
            srow = (q < 2 ? 0 : F) + fb * 64 + (q & 1) * 32 + (l & 31);
        }
        const uint16_t* src = blk + (at == FRAG_W2 ? 2 * fh : 0) + static_cast<int64_t>(srow) * K + k0;
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    }
}

// Round n fp32 values to bf16 with the same conversion the epilogues use.
__global__ void round_bf16_kernel(const float* __restrict__ in, uint16_t* __restrict__ out, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = f2bf(in[i]);
}

// Router probability on the FC1 input (paged-stash pull request, "What does
// this PR do": the optional multiply by the probability before FC1):
// out[r][h] = bf16(p_r x[r][h]), the fp32 product rounded to nearest even.
// One wavefront per row (four per workgroup, rows strided over the grid);
// lane l takes the row's 16-byte chunks l, l + 64, ...  x and out may be one
// buffer: a lane reads each chunk before it writes it.
__global__ __launch_bounds__(256) void scale_rows_kernel(const uint16_t* x, const float* __restrict__ probs,
                                                         int64_t M, int H, uint16_t* out) {
    const int lane = threadIdx.x & 63;
    const int nch = H / 8;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6); r < M;
         r += static_cast<int64_t>(gridDim.x) * 4) {
        const float p = probs[r];
        const uint16_t* xr = x + r * H;
        uint16_t* orow = out + r * H;
        for (int c = lane; c < nch; c += 64) {
            const uint4 v = *reinterpret_cast<const uint4*>(xr + c * 8);
            uint4 o;
            o.x = pack2(p * lo_f(v.x), p * hi_f(v.x));
            o.y = pack2(p * lo_f(v.y), p * hi_f(v.y));
            o.z = pack2(p * lo_f(v.z), p * hi_f(v.z));
            o.w = pack2(p * lo_f(v.w), p * hi_f(v.w));
            *reinterpret_cast<uint4*>(orow + c * 8) = o;
        }
    }
}

// Its input gradient, given g (the gradient at the scaled input) and the
// unscaled x: dx[r][h] = bf16(p_r g[r][h]) and dprobs[r] = sum_h g[r][h] x[r][h]
// in fp32 (products of two bf16 values are exact).  Lane l adds the products
// of its chunks l, l + 64, ... in increasing h; the 64 lane sums are then
// combined pairwise, lanes 32 apart first, so every row's sum has one fixed
// order.  dx may be g's buffer.
__global__ __launch_bounds__(256) void scale_rows_bwd_kernel(const uint16_t* g, const uint16_t* __restrict__ x,
                                                             const float* __restrict__ probs, int64_t M, int H,
                                                             uint16_t* dx, float* __restrict__ dprobs) {
    const int lane = threadIdx.x & 63;
    const int nch = H / 8;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6); r < M;
         r += static_cast<int64_t>(gridDim.x) * 4) {
        const float p = probs[r];
        const uint16_t* gr = g + r * H;
        const uint16_t* xr = x + r * H;
        uint16_t* drow = dx + r * H;
        float s = 0.f;
        for (int c = lane; c < nch; c += 64) {
            const uint4 gv = *reinterpret_cast<const uint4*>(gr + c * 8);
            const uint4 xv = *reinterpret_cast<const uint4*>(xr + c * 8);
            const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
            uint32_t ow[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float g0 = lo_f(gw[k]), g1 = hi_f(gw[k]);
                s += g0 * lo_f(xw[k]);
                s += g1 * hi_f(xw[k]);
                ow[k] = pack2(p * g0, p * g1);
            }
            *reinterpret_cast<uint4*>(drow + c * 8) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
        if (lane == 0 && dprobs) dprobs[r] = s;
    }
}

// dp of every routed row: the partial sums of its 32-column groups added in
// group order (the same order whichever flavor produced them).
__global__ void dp_reduce_kernel(const int64_t* __restrict__ offsets, int E, int M, const float* __restrict__ part,
                                 int ld, float* __restrict__ dprobs) {
    int64_t lo = offsets[0], hi = offsets[E];
    lo = lo < 0 ? 0 : (lo > M ? M : lo);
    hi = hi < lo ? lo : (hi > M ? M : hi);
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t r = lo + static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; r < hi; r += stride) {
        const float* pr = part + r * ld;
        float s = 0.0f;
        for (int g = 0; g < ld; ++g) s += pr[g];
        dprobs[r] = s;
    }
}

// ---------------------------------------------------------------- launchers

template <bool W_KN, int EPI, bool EXT>
static hipError_t launch_cfg(const GemmParams& p, int num_cu, hipStream_t stream) {
    constexpr int TILE_COLS = (EPI == EPI_SWIGLU) ? TBN / 2 : TBN;
    const int64_t tiles_n = (p.N + TILE_COLS - 1) / TILE_COLS;
    // Upper bound of sum_e ceil(m_e / TBM) without reading the offsets.
    const int64_t tiles_m_max = (static_cast<int64_t>(p.M) + static_cast<int64_t>(p.E) * (TBM - 1)) / TBM;
    const int64_t upper = tiles_m_max * tiles_n;
    int64_t grid = num_cu;            // one workgroup per CU (LDS-limited)
    if (upper < grid) grid = upper;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((grouped_gemm_kernel<W_KN, EPI, EXT>), dim3(static_cast<unsigned>(grid)), dim3(NTHREADS), 0,
                       stream, p);
    return hipGetLastError();
}

static bool plain_swiglu(const GemmParams& p) { return p.slope == 1.0f && !p.probs && !p.dp_part; }

// One four-wave launch: thin items, then tiles.  Grid: one workgroup per CU,
// or fewer when M and E bound the work below that.
template <int EPI, bool EXT>
static hipError_t launch_tile4(const GemmParams& p, int num_cu, hipStream_t stream) {
    constexpr int TILE_COLS = (EPI == EPI_SWIGLU) ? TBN / 2 : TBN;
    const int64_t tiles_n = p.N / TILE_COLS;
    // upper bound of sum_e ceil(m_e / 256) tiles, plus one thin item per expert and column block
    const int64_t tiles_m_max = (static_cast<int64_t>(p.M) + static_cast<int64_t>(p.E) * (TBM - 1)) / TBM;
    const int64_t work = (tiles_m_max + p.E) * tiles_n;
    const int64_t grid = work < num_cu ? work : num_cu;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((tile4_kernel<EPI, EXT>), dim3(static_cast<unsigned>(grid)), dim3(T4_THREADS), 0, stream, p);
    return hipGetLastError();
}

// With a fragment-ordered weight copy (p.wfrag) the whole GEMM is one
// four-wave launch; otherwise one eight-wave launch.
hipError_t launch_fc1_swiglu(const GemmParams& p, int num_cu, hipStream_t s) {
    const bool plain = plain_swiglu(p);
    if (!p.wfrag)
        return plain ? launch_cfg<false, EPI_SWIGLU, false>(p, num_cu, s)
                     : launch_cfg<false, EPI_SWIGLU, true>(p, num_cu, s);
    return plain ? launch_tile4<EPI_SWIGLU, false>(p, num_cu, s) : launch_tile4<EPI_SWIGLU, true>(p, num_cu, s);
}
hipError_t launch_fc2(const GemmParams& p, int num_cu, hipStream_t s) {
    if (!p.wfrag) return launch_cfg<false, EPI_STORE, false>(p, num_cu, s);
    return launch_tile4<EPI_STORE, false>(p, num_cu, s);
}
hipError_t launch_pack_frag(const uint16_t* packed, uint16_t* frag, int E, int H, int F, hipStream_t s) {
    const int64_t chunks = static_cast<int64_t>(E) * FRAG_BLOCK_FH * H * F / 8;
    int64_t blocks = (chunks + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(pack_frag_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, packed, frag, E, H,
                       F);
    return hipGetLastError();
}
// The SwiGLU derivative (plain, or with the slope, the row weights and dp)
// runs on four-wave tiles over W2^T's fragment copy when there is one and F
// is a multiple of the 256-column tile; every other shape on the eight-wave
// kernel (the same bits either way).
hipError_t launch_dgrad_fc2(const GemmParams& p, int num_cu, hipStream_t s) {
    if (p.wfrag && p.N % TBN == 0)
        return plain_swiglu(p) ? launch_tile4<EPI_DSWIGLU, false>(p, num_cu, s)
                               : launch_tile4<EPI_DSWIGLU, true>(p, num_cu, s);
    return plain_swiglu(p) ? launch_cfg<true, EPI_DSWIGLU, false>(p, num_cu, s)
                           : launch_cfg<true, EPI_DSWIGLU, true>(p, num_cu, s);
}
hipError_t launch_dgrad_fc1(const GemmParams& p, int num_cu, hipStream_t s) {
    if (!p.wfrag) return launch_cfg<true, EPI_STORE, false>(p, num_cu, s);
    return launch_tile4<EPI_STORE, false>(p, num_cu, s);   // W1^T fragments: the same K-contiguous form
}
hipError_t launch_dp_reduce(const int64_t* offsets, int E, int M, const float* part, int ld, float* dprobs,
                            hipStream_t s) {
    if (M <= 0) return hipSuccess;
    int64_t blocks = (static_cast<int64_t>(M) + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(dp_reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, offsets, E, M, part,
                       ld, dprobs);
    return hipGetLastError();
}
namespace {
unsigned row_blocks(int64_t M) {   // four rows per workgroup, at most 65536 workgroups
    const int64_t b = (M + 3) / 4;
    return static_cast<unsigned>(b < 65536 ? b : 65536);
}
}  // namespace

hipError_t launch_scale_rows(const uint16_t* x, const float* probs, int64_t M, int H, uint16_t* out,
                             hipStream_t s) {
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(scale_rows_kernel, dim3(row_blocks(M)), dim3(256), 0, s, x, probs, M, H, out);
    return hipGetLastError();
}

hipError_t launch_scale_rows_bwd(const uint16_t* g, const uint16_t* x, const float* probs, int64_t M, int H,
                                 uint16_t* dx, float* dprobs, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(scale_rows_bwd_kernel, dim3(row_blocks(M)), dim3(256), 0, s, g, x, probs, M, H, dx, dprobs);
    return hipGetLastError();
}

hipError_t launch_round_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(round_bf16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, in, out, n);
    return hipGetLastError();
}

}  // namespace gg
