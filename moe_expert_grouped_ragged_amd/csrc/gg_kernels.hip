// Grouped GEMM kernels for frozen MoE experts on CDNA4 (gfx950).
//
// One persistent launch covers every expert of a GEMM.  Each workgroup reads
// the int64 expert offsets from device memory, turns them into per-expert
// tile counts and an exclusive prefix sum in LDS (the per-expert sizes never
// go through the host, as in the TE device-metadata grouped GEMM pull
// request, section "Summary"), and then walks the global tile list.  Experts
// with no rows own no tiles, so their weights are never read.
//
// The tile core is a bf16 MFMA GEMM (v_mfma_f32_32x32x16_bf16, fp32
// accumulators) with both operands staged through LDS in a [row][k] layout
// whose 16-byte chunks are XOR-swizzled by row, double-buffered so the next
// K panel is loaded from HBM while the current one feeds the matrix cores.
// The weight side is the MFMA "A" operand and the token side the "B"
// operand, so each lane ends up holding one token row and four groups of
// four consecutive output columns: stores are 8-byte vectors.
//
// Variants (template parameter EPI and W_KN):
//   FC1 + SwiGLU  W_KN=false  weights W1_e [2F][H] (K-contiguous); a tile
//                 loads matching gate rows n.. and up rows F+n.. so SwiGLU
//                 is applied in registers; writes H1 (optional) and A.
//   FC2           W_KN=false  weights W2_e [H][F]; writes Y.
//   dgrad FC2     W_KN=true   dA = dY W2_e: the contraction runs over W2's
//                 rows, so the weight panel arrives [K][N] and is transposed
//                 in registers on its way into LDS; the epilogue applies the
//                 SwiGLU derivative with the saved H1 and writes dH1.
//   dgrad FC1     W_KN=true   dX = dH1 W1_e; writes dX.
// Rounding points mirror the unfused computation: H1, A, Y, dA, dH1 and dX
// are each rounded once to bf16 (round to nearest even); SwiGLU and its
// derivative read the rounded gate/up and dA.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gg_kernels.h"

namespace gg {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int BK = 64;          // K elements per LDS panel (128 bytes per row)
constexpr int CHUNKS = BK / 8;  // 16-byte chunks per panel row

__device__ __forceinline__ uint16_t f2bf(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ float bf2f(uint32_t b16) {
    return __builtin_bit_cast(float, b16 << 16);
}
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return static_cast<uint32_t>(f2bf(lo)) | (static_cast<uint32_t>(f2bf(hi)) << 16);
}

// Element offset of 16-byte chunk `ch` of panel row `row` (swizzled).
__device__ __forceinline__ int lds_off(int row, int ch) {
    return row * BK + ((ch ^ (row & 7)) << 3);
}

template <int NT>
__device__ __forceinline__ void build_schedule(const int64_t* __restrict__ offsets, int E, int M,
                                               int bm, int tiles_n, int* s_off, int* s_pre) {
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
        int sum = 0;
        for (int e = e0; e < e1; ++e) {
            const int m = max(0, s_off[e + 1] - s_off[e]);
            sum += ((m + bm - 1) / bm) * tiles_n;
        }
        int incl = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        int run = incl - sum;
        for (int e = e0; e < e1; ++e) {
            s_pre[e] = run;
            const int m = max(0, s_off[e + 1] - s_off[e]);
            run += ((m + bm - 1) / bm) * tiles_n;
        }
        if (lane == 63) s_pre[E] = incl;
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

template <int BM, int BN, int WAVES_M, int WAVES_N, bool W_KN, int EPI>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64)
void grouped_gemm_kernel(const GemmParams p) {
    constexpr int NT = WAVES_M * WAVES_N * 64;
    constexpr int WTM = BM / WAVES_M;           // token rows per wave
    constexpr int WTN = BN / WAVES_N;           // weight rows per wave
    constexpr int TM = WTM / 32;
    constexpr int TN = WTN / 32;
    constexpr int A_CHUNKS = BM * CHUNKS / NT;  // 16-byte token chunks per thread per panel
    constexpr int B_CHUNKS = BN * CHUNKS / NT;  // (K-contiguous weights)
    constexpr int B_BLOCKS = (BK / 4) * (BN / 8) / NT;  // 4x8 blocks per thread ([K][N] weights)
    static_assert(BM * CHUNKS % NT == 0 && BN * CHUNKS % NT == 0, "tile/threads");
    static_assert(!W_KN || ((BK / 4) * (BN / 8)) % NT == 0, "tile/threads");
    static_assert(EPI != EPI_SWIGLU || (TN % 2 == 0), "SwiGLU needs gate/up pairs per wave");

    __shared__ __attribute__((aligned(16))) uint16_t s_a[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t s_b[2][BN * BK];
    __shared__ int s_off[GG_KMAX_EXPERTS + 1];
    __shared__ int s_pre[GG_KMAX_EXPERTS + 1];

    const int E = p.E, M = p.M, K = p.K, N = p.N;
    // output columns covered by one tile
    constexpr int TILE_COLS = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const int tiles_n = (N + TILE_COLS - 1) / TILE_COLS;
    build_schedule<NT>(p.offsets, E, M, BM, tiles_n, s_off, s_pre);
    const int total = s_pre[E];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WAVES_N;
    const int wn = wave % WAVES_N;
    const int kiters = (K + BK - 1) / BK;

    // Workgroups are dealt round-robin over the 8 XCDs; give the workgroups of
    // one XCD consecutive tiles so that tiles sharing panels share an L2.
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int slot = (G % 8 == 0) ? (b & 7) * (G >> 3) + (b >> 3) : b;

    for (int t = slot; t < total; t += G) {
        const int e = find_expert(s_pre, E, t);
        const int local = t - s_pre[e];
        const int row_beg = s_off[e];
        const int row_end = s_off[e + 1];
        const int tiles_m = (row_end - row_beg + BM - 1) / BM;
        const int tm = local % tiles_m;
        const int tn = local / tiles_m;
        const int row0 = row_beg + tm * BM;
        const int col0 = tn * TILE_COLS;
        const uint16_t* __restrict__ w = p.w + static_cast<int64_t>(e) * p.w_expert_stride;
        const uint16_t* __restrict__ act = p.act;

        // ---- per-thread global source pointers for the token panel
        const uint16_t* a_src[A_CHUNKS];
        int a_kc[A_CHUNKS];
        int a_dst[A_CHUNKS];
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / CHUNKS, ch = idx % CHUNKS;
            const int grow = min(row0 + r, row_end - 1);
            a_src[i] = act + static_cast<int64_t>(grow) * K + ch * 8;
            a_kc[i] = ch * 8;
            a_dst[i] = lds_off(r, ch);
        }
        // ---- weight panel sources
        const uint16_t* b_src[W_KN ? B_BLOCKS : B_CHUNKS];
        int b_kc[W_KN ? B_BLOCKS : B_CHUNKS];
        int b_dst[W_KN ? B_BLOCKS : B_CHUNKS];
        if constexpr (!W_KN) {
#pragma unroll
            for (int i = 0; i < B_CHUNKS; ++i) {
                const int idx = tid + i * NT;
                const int r = idx / CHUNKS, ch = idx % CHUNKS;
                int wrow;
                if constexpr (EPI == EPI_SWIGLU) {
                    const int half = r / (BN / 2);
                    const int c = min(col0 + r % (BN / 2), N - 1);
                    wrow = c + half * p.up_off;
                } else {
                    wrow = min(col0 + r, N - 1);
                }
                b_src[i] = w + static_cast<int64_t>(wrow) * p.ldw + ch * 8;
                b_kc[i] = ch * 8;
                b_dst[i] = lds_off(r, ch);
            }
        } else {
#pragma unroll
            for (int i = 0; i < B_BLOCKS; ++i) {
                const int idx = tid + i * NT;
                const int kb = idx / (BN / 8), nb = idx % (BN / 8);
                const int c = min(col0 + nb * 8, N - 8);
                b_src[i] = w + static_cast<int64_t>(kb * 4) * p.ldw + c;
                b_kc[i] = kb * 4;
                b_dst[i] = nb * 8 * BK + kb * 4;   // row nb*8 (+cc), k = kb*4: swizzled below
            }
        }

        uint4 ra[A_CHUNKS];
        uint4 rb[W_KN ? B_BLOCKS * 4 : B_CHUNKS];

        auto load_panel = [&](int kt) {
            const int k0 = kt * BK;
#pragma unroll
            for (int i = 0; i < A_CHUNKS; ++i) {
                ra[i] = (k0 + a_kc[i] < K) ? *reinterpret_cast<const uint4*>(a_src[i] + k0)
                                           : make_uint4(0, 0, 0, 0);
            }
            if constexpr (!W_KN) {
#pragma unroll
                for (int i = 0; i < B_CHUNKS; ++i) {
                    rb[i] = (k0 + b_kc[i] < K) ? *reinterpret_cast<const uint4*>(b_src[i] + k0)
                                               : make_uint4(0, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int i = 0; i < B_BLOCKS; ++i) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int k = k0 + b_kc[i] + r;
                        rb[i * 4 + r] = (k < K) ? *reinterpret_cast<const uint4*>(
                                                      b_src[i] + static_cast<int64_t>(k0 + r) * p.ldw)
                                                : make_uint4(0, 0, 0, 0);
                    }
                }
            }
        };

        auto store_panel = [&](int buf) {
            uint16_t* sa = s_a[buf];
            uint16_t* sb = s_b[buf];
#pragma unroll
            for (int i = 0; i < A_CHUNKS; ++i) *reinterpret_cast<uint4*>(sa + a_dst[i]) = ra[i];
            if constexpr (!W_KN) {
#pragma unroll
                for (int i = 0; i < B_CHUNKS; ++i) *reinterpret_cast<uint4*>(sb + b_dst[i]) = rb[i];
            } else {
#pragma unroll
                for (int i = 0; i < B_BLOCKS; ++i) {
                    // rb[i*4 + r] holds row k = kb*4 + r, columns nb*8 .. nb*8+7.
                    const uint32_t* q0 = reinterpret_cast<const uint32_t*>(&rb[i * 4 + 0]);
                    const uint32_t* q1 = reinterpret_cast<const uint32_t*>(&rb[i * 4 + 1]);
                    const uint32_t* q2 = reinterpret_cast<const uint32_t*>(&rb[i * 4 + 2]);
                    const uint32_t* q3 = reinterpret_cast<const uint32_t*>(&rb[i * 4 + 3]);
                    const int nrow0 = b_dst[i] / BK;     // nb*8
                    const int kq = b_kc[i];              // kb*4
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        // column 2j (low halves) and 2j+1 (high halves)
                        uint2 lo, hi;
                        lo.x = (q0[j] & 0xffffu) | (q1[j] << 16);
                        lo.y = (q2[j] & 0xffffu) | (q3[j] << 16);
                        hi.x = (q0[j] >> 16) | (q1[j] & 0xffff0000u);
                        hi.y = (q2[j] >> 16) | (q3[j] & 0xffff0000u);
                        const int n_lo = nrow0 + 2 * j, n_hi = n_lo + 1;
                        const int ch = kq >> 3, sub = kq & 7;
                        *reinterpret_cast<uint2*>(sb + lds_off(n_lo, ch) + sub) = lo;
                        *reinterpret_cast<uint2*>(sb + lds_off(n_hi, ch) + sub) = hi;
                    }
                }
            }
        };

        f32x16 acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

        // weight-panel row of this wave's j-th 32-row fragment
        auto wfrag_row = [&](int j) -> int {
            if constexpr (EPI == EPI_SWIGLU) {
                constexpr int HALF = TN / 2;
                return (j < HALF) ? wn * (WTN / 2) + j * 32 : BN / 2 + wn * (WTN / 2) + (j - HALF) * 32;
            } else {
                return wn * WTN + j * 32;
            }
        };

        load_panel(0);
        store_panel(0);
        __syncthreads();
        for (int kt = 0; kt < kiters; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < kiters) load_panel(kt + 1);
            const uint16_t* sa = s_a[cur];
            const uint16_t* sb = s_b[cur];
#pragma unroll
            for (int s = 0; s < BK / 16; ++s) {
                const int ch = s * 2 + (lane >> 5);
                bf16x8 fa[TM], fb[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int r = wm * WTM + i * 32 + (lane & 31);
                    fa[i] = *reinterpret_cast<const bf16x8*>(sa + lds_off(r, ch));
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int r = wfrag_row(j) + (lane & 31);
                    fb[j] = *reinterpret_cast<const bf16x8*>(sb + lds_off(r, ch));
                }
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
            }
            if (kt + 1 < kiters) store_panel(cur ^ 1);
            __syncthreads();
        }

        // ---- epilogue: lane holds token row (lane & 31) of each token fragment and,
        // for register v, weight-panel row (v/4)*8 + (lane/32)*4 + v%4.
        const int cbase = (lane >> 5) * 4;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int grow = row0 + wm * WTM + i * 32 + (lane & 31);
            if (grow >= row_end) continue;
            if constexpr (EPI == EPI_STORE) {
                uint16_t* out = p.out0 + static_cast<int64_t>(grow) * N;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int c = col0 + wn * WTN + j * 32 + q * 8 + cbase;
                        if (c < N) {
                            uint2 v;
                            v.x = pack2(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]);
                            v.y = pack2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
                            *reinterpret_cast<uint2*>(out + c) = v;
                        }
                    }
                }
            } else if constexpr (EPI == EPI_SWIGLU) {
                constexpr int HALF = TN / 2;
                uint16_t* a_out = p.out0 + static_cast<int64_t>(grow) * N;
                uint16_t* h_out = p.out1 ? p.out1 + static_cast<int64_t>(grow) * (2 * N) : nullptr;
#pragma unroll
                for (int j = 0; j < HALF; ++j) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int c = col0 + wn * (WTN / 2) + j * 32 + q * 8 + cbase;
                        if (c < N) {
                            uint16_t gb[4], ub[4], ab[4];
#pragma unroll
                            for (int x = 0; x < 4; ++x) {
                                gb[x] = f2bf(acc[i][j][q * 4 + x]);
                                ub[x] = f2bf(acc[i][j + HALF][q * 4 + x]);
                                const float g = bf2f(gb[x]);
                                const float u = bf2f(ub[x]);
                                const float s = g / (1.0f + __expf(-g));
                                ab[x] = f2bf(s * u);
                            }
                            uint2 va, vg, vu;
                            va.x = ab[0] | (uint32_t(ab[1]) << 16);
                            va.y = ab[2] | (uint32_t(ab[3]) << 16);
                            *reinterpret_cast<uint2*>(a_out + c) = va;
                            if (h_out) {
                                vg.x = gb[0] | (uint32_t(gb[1]) << 16);
                                vg.y = gb[2] | (uint32_t(gb[3]) << 16);
                                vu.x = ub[0] | (uint32_t(ub[1]) << 16);
                                vu.y = ub[2] | (uint32_t(ub[3]) << 16);
                                *reinterpret_cast<uint2*>(h_out + c) = vg;
                                *reinterpret_cast<uint2*>(h_out + N + c) = vu;
                            }
                        }
                    }
                }
            } else {  // EPI_DSWIGLU: N == F, aux = H1 [M][2F], out0 = dH1 [M][2F]
                const uint16_t* h1 = p.aux + static_cast<int64_t>(grow) * (2 * N);
                uint16_t* dh = p.out0 + static_cast<int64_t>(grow) * (2 * N);
#pragma unroll
                for (int j = 0; j < TN; ++j) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int c = col0 + wn * WTN + j * 32 + q * 8 + cbase;
                        if (c < N) {
                            const uint2 hg = *reinterpret_cast<const uint2*>(h1 + c);
                            const uint2 hu = *reinterpret_cast<const uint2*>(h1 + N + c);
                            const uint32_t gw[2] = {hg.x, hg.y};
                            const uint32_t uw[2] = {hu.x, hu.y};
                            float dg[4], du[4];
#pragma unroll
                            for (int x = 0; x < 4; ++x) {
                                const uint32_t gbits = (x & 1) ? (gw[x >> 1] >> 16) : (gw[x >> 1] & 0xffffu);
                                const uint32_t ubits = (x & 1) ? (uw[x >> 1] >> 16) : (uw[x >> 1] & 0xffffu);
                                const float g = bf2f(gbits);
                                const float u = bf2f(ubits);
                                const float da = bf2f(f2bf(acc[i][j][q * 4 + x]));
                                const float s = 1.0f / (1.0f + __expf(-g));
                                dg[x] = da * u * s * (1.0f + g * (1.0f - s));
                                du[x] = da * g * s;
                            }
                            uint2 vg, vu;
                            vg.x = pack2(dg[0], dg[1]);
                            vg.y = pack2(dg[2], dg[3]);
                            vu.x = pack2(du[0], du[1]);
                            vu.y = pack2(du[2], du[3]);
                            *reinterpret_cast<uint2*>(dh + c) = vg;
                            *reinterpret_cast<uint2*>(dh + N + c) = vu;
                        }
                    }
                }
            }
        }
    }
}

// Round n fp32 values to bf16 with the same conversion the epilogues use.
__global__ void round_bf16_kernel(const float* __restrict__ in, uint16_t* __restrict__ out, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = f2bf(in[i]);
}

// ---------------------------------------------------------------- launchers

template <int BM, int BN, int WAVES_M, int WAVES_N, bool W_KN, int EPI>
static hipError_t launch_cfg(const GemmParams& p, int num_cu, hipStream_t stream) {
    constexpr int TILE_COLS = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const int64_t tiles_n = (p.N + TILE_COLS - 1) / TILE_COLS;
    // Upper bound of sum_e ceil(m_e / BM) without reading the offsets.
    const int64_t tiles_m_max = (static_cast<int64_t>(p.M) + static_cast<int64_t>(p.E) * (BM - 1)) / BM;
    const int64_t upper = tiles_m_max * tiles_n;
    int64_t grid = num_cu;            // one workgroup per CU (LDS-limited)
    if (upper < grid) grid = upper;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, BN, WAVES_M, WAVES_N, W_KN, EPI>),
                       dim3(static_cast<unsigned>(grid)), dim3(WAVES_M * WAVES_N * 64), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_fc1_swiglu(const GemmParams& p, int num_cu, hipStream_t s) {
    return launch_cfg<256, 256, 2, 4, false, EPI_SWIGLU>(p, num_cu, s);
}
hipError_t launch_fc2(const GemmParams& p, int num_cu, hipStream_t s) {
    return launch_cfg<256, 256, 2, 4, false, EPI_STORE>(p, num_cu, s);
}
hipError_t launch_dgrad_fc2(const GemmParams& p, int num_cu, hipStream_t s) {
    return launch_cfg<256, 256, 2, 4, true, EPI_DSWIGLU>(p, num_cu, s);
}
hipError_t launch_dgrad_fc1(const GemmParams& p, int num_cu, hipStream_t s) {
    return launch_cfg<256, 256, 2, 4, true, EPI_STORE>(p, num_cu, s);
}
hipError_t launch_round_bf16(const float* in, uint16_t* out, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(round_bf16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, in, out, n);
    return hipGetLastError();
}

}  // namespace gg
