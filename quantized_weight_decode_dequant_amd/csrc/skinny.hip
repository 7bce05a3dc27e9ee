// Skinny Q4 products Y[M, N] = X[M, K] W^T for M = 1..32 bf16 activation
// rows against weights streamed once per call: the verification pass of a
// 16-32 token draft (Uzu page, fange-kb.cn, section "Producing several tokens
// from one model pass": sixteen candidate rows give the matrix units sixteen
// rows of work instead of one).  The kernel runs on the gfx950 MFMA units
// with the 16x16x32 bf16 shape, whose B operand (lane l: 8 consecutive k of
// column l & 15, k-slice l >> 4) is exactly one packed weight slot (see
// qg_internal.h): each packed word becomes the bf16x8 operand (128 + q); one
// MFMA pair covers one group of 64, its fp32 result is scaled per (row n,
// group) on the VALU: acc += s * C + (b - 128 s) * sum_{k in g} X[m, k].
//
// The X slices staged in LDS have rows padded by 16 bytes so the 16
// A-operand rows of one MFMA hit distinct banks; see sk_q4_range for the work
// split.  This kernel serves single matrices too small to fill the chip with
// the streaming kernel of q4_skinny_stream.hip; the int8 path lives in
// q8_skinny.hip.
#include "qg_internal.h"

namespace qg {

constexpr int SK_WAVES = 4;
constexpr int SK_THREADS = SK_WAVES * 64;

// Q4 skinny, work split: a workgroup owns a contiguous range of rowblocks
// and walks it in blocks of SK_BLOCK = 4 * RPI * NI rowblocks.  For each
// K-segment of TPS tiles it stages that slice of X (all M rows) and its group
// sums in LDS once, then each wave sweeps NI iterations of RPI rowblocks: it
// loads their TPS tiles (8 slots per iteration), and accumulates the MFMA
// results into per-rowblock registers.  X is re-staged once per block and
// segment, not once per rowblock.  X is zero past K, so tiles past the end of
// K (clamped re-reads) contribute exactly zero; rowblocks past the range are
// computed from clamped re-reads and simply not stored.
template <int MT, int TPS, int RPI, int NI>
struct SkCfg {
    static constexpr int MP = MT * 16;          // padded rows of X
    static constexpr int RS = TPS * 128 + 8;    // LDS row stride in bf16 (16-byte pad)
    static constexpr int BLOCK = SK_WAVES * RPI * NI;
    static constexpr size_t LDS = (size_t)MP * RS * 2 + (size_t)2 * TPS * MP * 4;
};

template <int MT, int TPS, int RPI, int NI>
__device__ __forceinline__ void sk_q4_range(const WorkItem &it, int u0, int u1, int M,
                                            uint16_t *xl, float *xs, int tid,
                                            const Q4Consts &kq) {
    typedef SkCfg<MT, TPS, RPI, NI> C;
    constexpr int MP = C::MP, RS = C::RS;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), kg = lane >> 4;
    const int P = it.P, K = it.K, N = it.N;
    const int nseg = (P + TPS - 1) / TPS;
    const uint16_t *X = reinterpret_cast<const uint16_t *>(it.x);
    const unsigned lc = 16u * lane, ls = 1024u + 8u * (lane & 15);
#pragma unroll 1
    for (int ub = u0; ub < u1; ub += C::BLOCK) {
        f32x4_t acc[NI][RPI][MT];
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int r = 0; r < RPI; ++r)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[i][r][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int seg = 0; seg < nseg; ++seg) {
            const int p0 = seg * TPS, pn = min(TPS, P - p0);
            __syncthreads();  // the previous segment's LDS reads are done
            {
                constexpr int TOT = MP * TPS * 16;  // uint4 of the segment
                constexpr int U = (TOT + SK_THREADS - 1) / SK_THREADS;
                const int k0 = p0 * 128;
                u32x4_t v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int i = tid + u * SK_THREADS;
                    const int m = i / (TPS * 16), c8 = i % (TPS * 16);
                    const int k = k0 + c8 * 8;
                    v[u] = (i < TOT && m < M && k < K)
                               ? ld_global(reinterpret_cast<const u32x4_t *>(X + (size_t)m * K + k))
                               : u32x4_t{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int i = tid + u * SK_THREADS;
                    const int m = i / (TPS * 16), c8 = i % (TPS * 16);
                    if (i < TOT) *reinterpret_cast<u32x4_t *>(xl + m * RS + c8 * 8) = v[u];
                }
            }
            __syncthreads();
            for (int i = tid; i < 2 * TPS * MP; i += SK_THREADS) {
                const int g = i / MP, m = i % MP;
                const uint4 *rr = reinterpret_cast<const uint4 *>(xl + m * RS + g * 64);
                float sum = 0.f;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const uint4 w = rr[q];
                    sum += bf16_lo(w.x) + bf16_hi(w.x) + bf16_lo(w.y) + bf16_hi(w.y) + bf16_lo(w.z) +
                           bf16_hi(w.z) + bf16_lo(w.w) + bf16_hi(w.w);
                }
                xs[i] = sum;
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                // this iteration's RPI rowblocks, TPS tiles each
                u32x4_t c[TPS][RPI];
                u32x2_t sb[TPS][RPI];
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int r = 0; r < RPI; ++r) {
                    const int rb = min(ub + (i * SK_WAVES + wave) * RPI + r, u1 - 1);
                    const __amdgpu_buffer_rsrc_t rs =
                        make_rsrc(uniform_ptr(it.packed + ((size_t)rb * P + p0) * Q4_TILE_BYTES),
                                  (unsigned)pn * Q4_TILE_BYTES);
#pragma unroll
                    for (int j = 0; j < TPS; ++j) {
                        const unsigned to = (unsigned)min(j, pn - 1) * Q4_TILE_BYTES;
                        c[j][r] = buf_ld_x4(rs, lc, to);
                        sb[j][r] = buf_ld_x2(rs, ls, to);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < TPS; ++j) {
                    // one tile's operands live at a time (the scheduler would
                    // otherwise hoist every tile's LDS reads and spill)
                    __builtin_amdgcn_sched_barrier(0);
                    bf16x8_t A[MT][4];
                    f32x4_t xs0[MT], xs1[MT];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const uint16_t *ar = xl + (16 * mt + (lane & 15)) * RS + j * 128 + 8 * kg;
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            A[mt][q] = *reinterpret_cast<const bf16x8_t *>(ar + 32 * q);
                        xs0[mt] = *reinterpret_cast<const f32x4_t *>(xs + (2 * j) * MP + 16 * mt + 4 * kg);
                        xs1[mt] = *reinterpret_cast<const f32x4_t *>(xs + (2 * j + 1) * MP + 16 * mt + 4 * kg);
                    }
#pragma unroll
                    for (int r = 0; r < RPI; ++r) {
                        bf16x8_t B[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) B[q] = q4_word_to_bf16x8(c[j][r][q], kq);
                        const float s0 = f16_lo(sb[j][r][0]), b0 = f16_hi(sb[j][r][0]);
                        const float s1 = f16_lo(sb[j][r][1]), b1 = f16_hi(sb[j][r][1]);
                        const float bb0 = fmaf(-128.f, s0, b0), bb1 = fmaf(-128.f, s1, b1);
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
                            f32x4_t C0 = {0.f, 0.f, 0.f, 0.f}, C1 = {0.f, 0.f, 0.f, 0.f};
                            C0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][0], B[0], C0, 0, 0, 0);
                            C0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][1], B[1], C0, 0, 0, 0);
                            C1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][2], B[2], C1, 0, 0, 0);
                            C1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][3], B[3], C1, 0, 0, 0);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                float a = acc[i][r][mt][e];
                                a = fmaf(s0, C0[e], a);
                                a = fmaf(bb0, xs0[mt][e], a);
                                a = fmaf(s1, C1[e], a);
                                a = fmaf(bb1, xs1[mt][e], a);
                                acc[i][r][mt][e] = a;
                            }
                        }
                    }
                }
            }
        }
        // the block's outputs: each wave stores its own rowblocks
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int r = 0; r < RPI; ++r) {
                const int rb = ub + (i * SK_WAVES + wave) * RPI + r;
                const int n = rb * RB + (lane & 15);
                if (rb < u1 && n < N) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int m = 16 * mt + 4 * kg + e;
                            if (m < M) {
                                if (it.out_f32)
                                    st_global<float>(it.y, (size_t)m * N + n, acc[i][r][mt][e]);
                                else
                                    st_global<uint16_t>(it.y, (size_t)m * N + n,
                                                        f32_to_bf16(acc[i][r][mt][e]));
                            }
                        }
                }
            }
    }
}

// <MT, TPS, RPI, NI, workgroups per CU>.  M <= 16: one 16-row tile, 8 tiles
// (1024 k) per segment, blocks of 24 rowblocks, 166 VGPRs (3 workgroups per
// CU); M <= 32: two 16-row tiles, 4 tiles per segment, blocks of 16
// rowblocks, 2 workgroups per CU.  Both stage 33 KB of X per segment; the
// register budgets are the largest that compile without spilling.
#define SK_M16 1, 8, 1, 6, 3
#define SK_M32 2, 4, 1, 4, 2

template <int MT, int TPS, int RPI, int NI, int WPC>
__global__ void __launch_bounds__(SK_THREADS, WPC)
q4_skinny_kernel(WorkItem it, int M) {
    typedef SkCfg<MT, TPS, RPI, NI> C;
    __shared__ __attribute__((aligned(16))) uint16_t xl[C::MP * C::RS];
    __shared__ __attribute__((aligned(16))) float xs[2 * TPS * C::MP];  // [group-in-segment][m]
    const Q4Consts kq = q4_consts();
    const int64_t n = it.units, g = gridDim.x, j = blockIdx.x;
    const int u0 = (int)(j * n / g), u1 = (int)((j + 1) * n / g);
    if (u0 < u1) sk_q4_range<MT, TPS, RPI, NI>(it, u0, u1, M, xl, xs, (int)threadIdx.x, kq);
}

static inline int min_grid(int units, int cap) { return units < cap ? units : cap; }

static int q4_skinny_wgs_per_cu(int64_t M) { return M <= 16 ? 3 : 2; }

hipError_t launch_q4_skinny(const uint8_t *packed, const uint16_t *X, void *Y, int64_t M,
                            int64_t N, int64_t K, bool out_f32, int cus, hipStream_t s) {
    WorkItem it{};
    it.packed = packed;
    it.x = X;
    it.y = Y;
    it.N = (int32_t)N;
    it.K = (int32_t)K;
    it.P = (int32_t)ceil_div(K, Q4_TILE_K);
    it.units = (int32_t)ceil_div(N, RB);
    it.out_f32 = out_f32 ? 1 : 0;
    // blocks of 32 rowblocks unless that leaves CUs idle
    const int grid = min_grid((int)ceil_div(it.units, 8), cus * q4_skinny_wgs_per_cu(M));
    if (M <= 16)
        hipLaunchKernelGGL((q4_skinny_kernel<SK_M16>), dim3(grid), dim3(SK_THREADS), 0, s, it,
                           (int)M);
    else
        hipLaunchKernelGGL((q4_skinny_kernel<SK_M32>), dim3(grid), dim3(SK_THREADS), 0, s, it,
                           (int)M);
    return hipGetLastError();
}

}  // namespace qg
