// Q8 skinny product on the int8 matrix path: activations already rotated by
// the block-diagonal randomized Hadamard-32 and quantized per row to int8
// (Xq, scale sx[m]); weights 8-bit symmetric with an fp16 scale per group of
// 32 (Uzu page, fange-kb.cn, section "How Uzu optimizes bytes and tokens per
// pass": verification runs on int8 activations against 8-bit weights).
//
//   Y[m, n] = sx[m] * sum_g sw[n, g] * P[m, n, g],
//   P[m, n, g] = sum_{k in g} Xq[m, k] * Wq[n, k]   (exact int32).
//
// One v_mfma_i32_16x16x32_i8 per group of 32 yields P for 16 activation rows
// x 16 weight rows; its B operand (lane l: 8 consecutive k of row l & 15,
// k-slice l >> 4) is half of one 16-byte packed slot (see qg_internal.h).
//
// Work split.  A call streams every weight byte once, and a single matrix of
// this pass is only tens of MB, so the launch must put the whole chip's load
// queue to work at once rather than stream a few rowblocks per CU.  A
// workgroup owns one rowblock (16 weight rows) at a time and its W waves
// split that rowblock's K: wave w takes chunks w, w + W, ... of T tiles (128
// k each), issues all of a chunk's weight loads and the matching Xq loads
// (the MFMA A operand, read straight from the L2-resident activation tile)
// before any arithmetic, then folds the group partials into fp32.  The W
// per-wave partial sums are reduced in LDS in wave order (deterministic) and
// the first MT waves write Y.  Loads go through buffer resources: Xq rows
// past M read as zero; chunk slots past the rowblock's last tile re-read
// that tile and are given a zero scale (their int32 partials are finite, so
// the fp32 sums are unchanged) and never write group partials.
#include "qg_internal.h"

namespace qg {

constexpr int Q8_WMAX = 16;  // waves per workgroup

template <int MT, int T, bool GROUPS>
__global__ void __launch_bounds__(Q8_WMAX * 64)
q8_skinny_kernel(const uint8_t *__restrict__ packed, const int8_t *__restrict__ X,
                 const float *__restrict__ x_scales, void *__restrict__ Y, int M, int N, int K,
                 int P, int nrb, int out_f32) {
    __shared__ f32x4_t red[GROUPS ? 1 : Q8_WMAX][MT][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int W = blockDim.x >> 6;
    const int kg = lane >> 4, r16 = lane & 15;
    const int G = K / 32;
    const int nch = (P + T - 1) / T;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (unsigned)(M * K));
    // Xq row of this lane in each 16-row activation tile; rows >= M start
    // at or past M * K and read as zero
    unsigned xo[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xo[mt] = (unsigned)((16 * mt + r16) * K + 8 * kg);
    const unsigned wbytes = (unsigned)P * Q8_TILE_BYTES;

#pragma unroll 1
    for (int rb = blockIdx.x; rb < nrb; rb += gridDim.x) {
        const __amdgpu_buffer_rsrc_t rw =
            make_rsrc(uniform_ptr(packed + (size_t)rb * wbytes), wbytes);
        const int n = rb * RB + r16;
        f32x4_t acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int c = wave; c < nch; c += W) {
            const int p0 = c * T;
            u32x4_t c0[T], c1[T];
            u32x2_t sc[T], a[T][4][MT];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < T; ++j) {
                // tiles past the end re-read the last tile (their scales
                // are zeroed below); the uniform tile offset rides in soffset
                const unsigned tw = (unsigned)min(p0 + j, P - 1) * Q8_TILE_BYTES;
                c0[j] = buf_ld_x4(rw, 16u * lane, tw);
                c1[j] = buf_ld_x4(rw, 16u * lane + 1024u, tw);
                sc[j] = buf_ld_x2(rw, 8u * r16 + 2048u, tw);
            }
#pragma unroll
            for (int j = 0; j < T; ++j) {
                // the whole Xq offset in the range-checked VGPR offset
                const unsigned tx = (unsigned)min(p0 + j, P - 1) * 128u;
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        a[j][g][mt] = buf_ld_x2(rx, xo[mt] + tx + 32u * g, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < T; ++j) {
                // one tile's partials live at a time
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const u32x4_t &ch = (g < 2) ? c0[j] : c1[j];
                    const u32x2_t bw = {ch[2 * (g & 1)], ch[2 * (g & 1) + 1]};
                    const long bop = __builtin_bit_cast(long, bw);
                    const unsigned swbits = sc[j][g >> 1];
                    const float sw = (p0 + j < P) ? ((g & 1) ? f16_hi(swbits) : f16_lo(swbits)) : 0.f;
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const long aop = __builtin_bit_cast(long, a[j][g][mt]);
                        const i32x4_t C = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                            aop, bop, i32x4_t{0, 0, 0, 0}, 0, 0, 0);
                        if constexpr (GROUPS) {
                            const int gg = (p0 + j) * 4 + g;
                            if (gg < G && n < N) {
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    const int m = 16 * mt + 4 * kg + e;
                                    if (m < M)
                                        reinterpret_cast<int32_t *>(Y)[((size_t)m * N + n) * G + gg] = C[e];
                                }
                            }
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e) acc[mt][e] = fmaf(sw, (float)C[e], acc[mt][e]);
                        }
                    }
                }
            }
        }
        if constexpr (!GROUPS) {
            // K-split reduction over the waves, in wave order
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) red[wave][mt][lane] = acc[mt];
            __syncthreads();
#pragma unroll 1
            for (int mt = wave; mt < MT; mt += W) {
                f32x4_t s = red[0][mt][lane];
#pragma unroll 1
                for (int w = 1; w < W; ++w) s += red[w][mt][lane];
                if (n < N) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int m = 16 * mt + 4 * kg + e;
                        if (m < M) {
                            const float v = x_scales[m] * s[e];
                            if (out_f32)
                                reinterpret_cast<float *>(Y)[(size_t)m * N + n] = v;
                            else
                                reinterpret_cast<uint16_t *>(Y)[(size_t)m * N + n] = f32_to_bf16(v);
                        }
                    }
                }
            }
            __syncthreads();  // red is reused by the next rowblock
        }
    }
}

// Tiles per wave chunk: the smallest compiled size with which 16 waves cover
// the rowblock's K in one chunk each, so every weight byte of a rowblock is
// requested at the start; longer K loops.  The register budget (1024-thread
// workgroups leave 128 VGPRs per lane) caps T at 6 for one 16-row activation
// tile and 4 for two (T = 6 spills a few registers that are only reloaded by
// the epilogue).
template <int MT, bool GROUPS>
static hipError_t launch_q8_mt(const uint8_t *packed, const int8_t *X, const float *x_scales,
                               void *Y, int M, int N, int K, int P, int nrb, int out_f32,
                               hipStream_t s) {
    const int need = (P + Q8_WMAX - 1) / Q8_WMAX;
    int T = MT == 1 ? 6 : 4;
    if (need <= 2 || GROUPS) T = 2;  // the group-partial mode is for testing
    else if (need <= 4) T = 4;
    const int nch = (P + T - 1) / T;
    const int W = nch < Q8_WMAX ? nch : Q8_WMAX;
    const int grid = nrb < 65536 ? nrb : 65536;
    const dim3 g(grid), b(W * 64);
    if (GROUPS || T == 2)
        hipLaunchKernelGGL((q8_skinny_kernel<MT, 2, GROUPS>), g, b, 0, s, packed, X, x_scales, Y, M,
                           N, K, P, nrb, out_f32);
    else if (T == 4)
        hipLaunchKernelGGL((q8_skinny_kernel<MT, 4, false>), g, b, 0, s, packed, X, x_scales, Y, M,
                           N, K, P, nrb, out_f32);
    else
        hipLaunchKernelGGL((q8_skinny_kernel<MT, (MT == 1 ? 6 : 4), false>), g, b, 0, s, packed, X,
                           x_scales, Y, M, N, K, P, nrb, out_f32);
    return hipGetLastError();
}

hipError_t launch_q8_skinny(const uint8_t *packed, const int8_t *X, const float *x_scales,
                            void *Y, int64_t M, int64_t N, int64_t K, int out_mode, int cus,
                            hipStream_t s) {
    (void)cus;
    const int P = (int)ceil_div(K, Q8_TILE_K);
    const int nrb = (int)ceil_div(N, RB);
    const int f32 = out_mode == 1 ? 1 : 0;
    if (out_mode == 2)
        return M <= 16 ? launch_q8_mt<1, true>(packed, X, x_scales, Y, (int)M, (int)N, (int)K, P, nrb, 0, s)
                       : launch_q8_mt<2, true>(packed, X, x_scales, Y, (int)M, (int)N, (int)K, P, nrb, 0, s);
    return M <= 16 ? launch_q8_mt<1, false>(packed, X, x_scales, Y, (int)M, (int)N, (int)K, P, nrb, f32, s)
                   : launch_q8_mt<2, false>(packed, X, x_scales, Y, (int)M, (int)N, (int)K, P, nrb, f32, s);
}

}  // namespace qg
