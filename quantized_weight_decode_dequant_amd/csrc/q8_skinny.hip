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
// Work split.  A single matrix of this pass is only tens of MB and its
// activation tile is 64-384 KB, so the launch gives every CU one workgroup
// of 16 waves, which holds a K-segment of Xq (up to 96 KB) in LDS and walks
// rowblocks (16 weight rows) in a grid-strided loop.  Within a rowblock the
// 16 waves split K: wave w takes T consecutive 128-k tiles of each segment.
// The weight loads of a rowblock are all issued at once, right after the
// first Xq loads of the segment (see q8_stage_pre); when K is one segment
// those of the next rowblock go out before the arithmetic of the current
// one.  Xq is staged with coalesced 16-byte loads and read back by each MFMA
// as its 8-byte A operand.  The 16 per-wave partial sums of a rowblock are
// reduced in LDS in wave order (deterministic).  Weight tiles past the end of K read
// as zero (their offsets sit in the range-checked part of the buffer
// address), and so does Xq past K and past row M, so ragged shapes need no
// branches.
#include "qg_internal.h"

namespace qg {

constexpr int Q8_WAVES = 16;
constexpr int Q8_THREADS = Q8_WAVES * 64;

template <int MT, int T>
struct Q8Cfg {
    static constexpr int MP = 16 * MT;                // padded activation rows
    static constexpr int SEGT = Q8_WAVES * T;         // tiles per staged segment
    static constexpr int RS = SEGT * Q8_TILE_K + 8;   // LDS row stride in bytes (8 mod 128)
    static constexpr size_t LDS_X = (size_t)MP * RS;
};

template <int T>
struct Q8W {
    u32x4_t c0[T], c1[T];
    u32x2_t sc[T];
};

// The loads of tiles [p0, p0 + T) of one rowblock (buffer rw over its P
// tiles; an empty buffer, or tiles past P, read as zero).
template <int T>
__device__ __forceinline__ void q8_load(Q8W<T> &B, __amdgpu_buffer_rsrc_t rw, int p0, int lane) {
    const unsigned lc = 16u * lane, ls = 2048u + 8u * (lane & 15);
#pragma unroll
    for (int j = 0; j < T; ++j) {
        const unsigned tw = (unsigned)(p0 + j) * Q8_TILE_BYTES;
        B.c0[j] = buf_ld_x4(rw, tw + lc, 0);
        B.c1[j] = buf_ld_x4(rw, tw + lc + 1024u, 0);
        B.sc[j] = buf_ld_x2(rw, tw + ls, 0);
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t q8_rsrc(const uint8_t *packed, int rb, int P,
                                                          bool valid) {
    const unsigned wbytes = (unsigned)P * Q8_TILE_BYTES;
    return make_rsrc(uniform_ptr(packed + (size_t)rb * wbytes), valid ? wbytes : 0u);
}

// Staging of segment `seg` of Xq (SEGT tiles; zero past K and past row M).
// The first Q8_PRE 16-byte chunks per thread are loaded into registers by
// q8_stage_pre, which callers issue before the segment's weight loads (a
// wave's loads complete in issue order, so Xq loaded after the weights would
// wait for them); q8_stage_rest stores them, stages the remaining chunks, if
// any, and ends with a barrier.
constexpr int Q8_PRE = 4;

template <int MT, int T>
struct Q8Stage {
    static constexpr int PER_ROW = Q8Cfg<MT, T>::SEGT * Q8_TILE_K / 16;  // 16-byte chunks per row
    static constexpr int TOTAL = Q8Cfg<MT, T>::MP * PER_ROW;
    u32x4_t v[Q8_PRE];
};

template <int MT, int T>
__device__ __forceinline__ u32x4_t q8_chunk(const int8_t *X, int M, int K, int seg, int i) {
    typedef Q8Stage<MT, T> S;
    const int m = i / S::PER_ROW, c = i - m * S::PER_ROW;
    const int k = seg * Q8Cfg<MT, T>::SEGT * Q8_TILE_K + 16 * c;
    return (i < S::TOTAL && m < M && k < K)
               ? ld_global(reinterpret_cast<const u32x4_t *>(X + (size_t)m * K + k))
               : u32x4_t{0u, 0u, 0u, 0u};
}

template <int MT, int T>
__device__ __forceinline__ void q8_chunk_store(int8_t *xl, int i, u32x4_t v) {
    typedef Q8Stage<MT, T> S;
    const int m = i / S::PER_ROW, c = i - m * S::PER_ROW;
    if (i < S::TOTAL) {
        // rows are 8-byte aligned: two 8-byte stores
        u32x2_t *d = reinterpret_cast<u32x2_t *>(xl + m * Q8Cfg<MT, T>::RS + 16 * c);
        d[0] = u32x2_t{v[0], v[1]};
        d[1] = u32x2_t{v[2], v[3]};
    }
}

template <int MT, int T>
__device__ __forceinline__ void q8_stage_pre(Q8Stage<MT, T> &st, const int8_t *X, int M, int K,
                                             int seg, int tid) {
#pragma unroll
    for (int u = 0; u < Q8_PRE; ++u) st.v[u] = q8_chunk<MT, T>(X, M, K, seg, tid + u * Q8_THREADS);
}

template <int MT, int T>
__device__ __forceinline__ void q8_stage_rest(const Q8Stage<MT, T> &st, const int8_t *X, int M,
                                              int K, int seg, int8_t *xl, int tid) {
    typedef Q8Stage<MT, T> S;
#pragma unroll
    for (int u = 0; u < Q8_PRE; ++u) q8_chunk_store<MT, T>(xl, tid + u * Q8_THREADS, st.v[u]);
    constexpr int U = 4;
#pragma unroll 1
    for (int i0 = tid + Q8_PRE * Q8_THREADS; i0 < S::TOTAL; i0 += U * Q8_THREADS) {
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = q8_chunk<MT, T>(X, M, K, seg, i0 + u * Q8_THREADS);
#pragma unroll
        for (int u = 0; u < U; ++u) q8_chunk_store<MT, T>(xl, i0 + u * Q8_THREADS, v[u]);
    }
    __syncthreads();
}

// The MFMAs of this wave's tiles (segment-relative index ps of its first
// tile, absolute index p0); group partials are either folded into acc with
// the weight scales or, for GROUPS, written out as they are.
template <int MT, int T, bool GROUPS>
__device__ __forceinline__ void q8_compute(const Q8W<T> &B, const int8_t *xl, int ps, int p0,
                                           int lane, f32x4_t acc[MT], void *Y, int M, int N,
                                           int G, int n) {
    typedef Q8Cfg<MT, T> C;
    const int kg = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int j = 0; j < T; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const u32x4_t &ch = (g < 2) ? B.c0[j] : B.c1[j];
            const u32x2_t bw = {ch[2 * (g & 1)], ch[2 * (g & 1) + 1]};
            const long bop = __builtin_bit_cast(long, bw);
            const unsigned swbits = B.sc[j][g >> 1];
            const float sw = (g & 1) ? f16_hi(swbits) : f16_lo(swbits);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const long aop = *reinterpret_cast<const long *>(
                    xl + (16 * mt + r16) * C::RS + (ps + j) * Q8_TILE_K + 32 * g + 8 * kg);
                const i32x4_t P4 = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop, i32x4_t{0, 0, 0, 0},
                                                                        0, 0, 0);
                if constexpr (GROUPS) {
                    const int gg = (p0 + j) * 4 + g;
                    if (gg < G && n < N) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int m = 16 * mt + 4 * kg + e;
                            if (m < M) st_global<int32_t>(Y, ((size_t)m * N + n) * G + gg, P4[e]);
                        }
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[mt][e] = fmaf(sw, (float)P4[e], acc[mt][e]);
                }
            }
        }
    }
}

// Sum the 16 waves' partials of rowblock rb in wave order and write Y.  xsc
// holds the row scales of this lane's output rows (m = 16 mt + 4 kg + e),
// read once at the start: a global load here would complete only after the
// weight loads issued before it (loads complete in issue order), so the
// reduction, and every wave waiting on it, would wait for the next
// rowblock's weights.  With DB (two reduction buffers fit in LDS) the
// partials of consecutive rowblocks alternate between the buffers, so one
// barrier per 16-row tile suffices (a buffer is written again only after
// the barrier of the next tile, which its readers pass after reading), and
// waves 0..3 each add one of a lane's four values and store it; without,
// wave 0 adds and stores all four between two barriers.  Either way every
// value is the same sum in the same order.
template <int MT, bool DB>
__device__ __forceinline__ void q8_finish(const f32x4_t acc[MT], f32x4_t (*red)[Q8_WAVES][64],
                                          int &par, int wave, int lane, const f32x4_t xsc[MT],
                                          void *Y, int M, int N, int n, int out_f32) {
    const int kg = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        f32x4_t(*rb)[64] = red[DB ? par : 0];
        rb[wave][lane] = acc[mt];
        __syncthreads();
        if (DB) {
            if (wave < 4) {
                const int e = wave, m = 16 * mt + 4 * kg + e;
                float v = rb[0][lane][e];
#pragma unroll
                for (int w = 1; w < Q8_WAVES; ++w) v += rb[w][lane][e];
                const float sc = e == 0 ? xsc[mt][0] : e == 1 ? xsc[mt][1] : e == 2 ? xsc[mt][2] : xsc[mt][3];
                if (n < N && m < M) {
                    if (out_f32)
                        st_global<float>(Y, (size_t)m * N + n, sc * v);
                    else
                        st_global<uint16_t>(Y, (size_t)m * N + n, f32_to_bf16(sc * v));
                }
            }
            par ^= 1;
        } else {
            if (wave == 0) {
                f32x4_t sum = rb[0][lane];
#pragma unroll
                for (int w = 1; w < Q8_WAVES; ++w) sum += rb[w][lane];
                if (n < N) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int m = 16 * mt + 4 * kg + e;
                        if (m < M) {
                            const float v = xsc[mt][e] * sum[e];
                            if (out_f32)
                                st_global<float>(Y, (size_t)m * N + n, v);
                            else
                                st_global<uint16_t>(Y, (size_t)m * N + n, f32_to_bf16(v));
                        }
                    }
                }
            }
            __syncthreads();
        }
    }
}

template <int MT>
__device__ __forceinline__ void q8_zero(f32x4_t a[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) a[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

template <int MT, int T, bool GROUPS>
__global__ void __launch_bounds__(Q8_THREADS, 1)
q8_skinny_kernel(const uint8_t *__restrict__ packed, const int8_t *__restrict__ X,
                 const float *__restrict__ x_scales, void *__restrict__ Y, int M, int N, int K,
                 int P, int nrb, int out_f32) {
    typedef Q8Cfg<MT, T> C;
    // two reduction buffers when they fit beside Xq
    constexpr bool DB = C::LDS_X + 2 * sizeof(f32x4_t) * Q8_WAVES * 64 <= 160 * 1024;
    __shared__ __attribute__((aligned(16))) int8_t xl[C::LDS_X];
    __shared__ f32x4_t red[GROUPS ? 1 : (DB ? 2 : 1)][GROUPS ? 1 : Q8_WAVES][64];
    int par = 0;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = K / 32;
    const int nseg = (P + C::SEGT - 1) / C::SEGT;
    int rb = blockIdx.x;
    if (rb >= nrb) return;
    // the scales of this lane's output rows, before any weight load
    f32x4_t xsc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 16 * mt + 4 * (lane >> 4) + e;
            xsc[mt][e] = (!GROUPS && m < M) ? x_scales[m] : 0.f;
        }
    f32x4_t acc[MT];
    Q8W<T> A, B;
    if (nseg == 1) {
        // Xq staged once; the next rowblock's weights load during this one's
        // arithmetic
        const int p0 = wave * T;
        Q8Stage<MT, T> st;
        q8_stage_pre<MT, T>(st, X, M, K, 0, tid);
        q8_load<T>(A, q8_rsrc(packed, rb, P, true), p0, lane);
        q8_stage_rest<MT, T>(st, X, M, K, 0, xl, tid);
#pragma unroll 1
        for (;;) {
            int nx = rb + gridDim.x;
            q8_load<T>(B, q8_rsrc(packed, nx, P, nx < nrb), p0, lane);
            __builtin_amdgcn_sched_barrier(0);
            q8_zero<MT>(acc);
            const int n = rb * RB + (lane & 15);
            q8_compute<MT, T, GROUPS>(A, xl, p0, p0, lane, acc, Y, M, N, G, n);
            if constexpr (!GROUPS) q8_finish<MT, DB>(acc, red, par, wave, lane, xsc, Y, M, N, n, out_f32);
            if (nx >= nrb) break;
            rb = nx;
            nx = rb + gridDim.x;
            q8_load<T>(A, q8_rsrc(packed, nx, P, nx < nrb), p0, lane);
            __builtin_amdgcn_sched_barrier(0);
            q8_zero<MT>(acc);
            const int n2 = rb * RB + (lane & 15);
            q8_compute<MT, T, GROUPS>(B, xl, p0, p0, lane, acc, Y, M, N, G, n2);
            if constexpr (!GROUPS) q8_finish<MT, DB>(acc, red, par, wave, lane, xsc, Y, M, N, n2, out_f32);
            if (nx >= nrb) break;
            rb = nx;
        }
        return;
    }
    // several segments per rowblock: Xq re-staged per segment, each
    // segment's weight loads issued before its staging
#pragma unroll 1
    for (; rb < nrb; rb += gridDim.x) {
        const int n = rb * RB + (lane & 15);
        q8_zero<MT>(acc);
#pragma unroll 1
        for (int seg = 0; seg < nseg; ++seg) {
            const int p0 = seg * C::SEGT + wave * T;
            Q8Stage<MT, T> st;
            q8_stage_pre<MT, T>(st, X, M, K, seg, tid);
            q8_load<T>(A, q8_rsrc(packed, rb, P, true), p0, lane);
            __syncthreads();  // nobody still reads the previous segment
            q8_stage_rest<MT, T>(st, X, M, K, seg, xl, tid);
            q8_compute<MT, T, GROUPS>(A, xl, wave * T, p0, lane, acc, Y, M, N, G, n);
        }
        if constexpr (!GROUPS) q8_finish<MT, DB>(acc, red, par, wave, lane, xsc, Y, M, N, n, out_f32);
    }
    (void)B;
}

// Tiles per wave and segment: fewest segments first, then least padding.
template <int MT>
static int q8_pick_t(int P) {
    const int cands1[2] = {2, 3}, cands2[2] = {1, 2};
    const int *c = MT == 1 ? cands1 : cands2;
    const int nc = 2;
    int best = c[0], bseg = 1 << 30, bwaste = 1 << 30;
    for (int i = 0; i < nc; ++i) {
        const int segt = Q8_WAVES * c[i];
        const int nseg = (P + segt - 1) / segt, waste = nseg * segt - P;
        if (nseg < bseg || (nseg == bseg && waste < bwaste)) {
            best = c[i];
            bseg = nseg;
            bwaste = waste;
        }
    }
    return best;
}

template <int MT, int T, bool GROUPS>
static void q8_launch(int grid, hipStream_t s, const uint8_t *packed, const int8_t *X,
                      const float *x_scales, void *Y, int M, int N, int K, int P, int nrb,
                      int out_f32) {
    hipLaunchKernelGGL((q8_skinny_kernel<MT, T, GROUPS>), dim3(grid), dim3(Q8_THREADS), 0, s,
                       packed, X, x_scales, Y, M, N, K, P, nrb, out_f32);
}

template <int MT, bool GROUPS>
static hipError_t launch_q8_mt(const uint8_t *packed, const int8_t *X, const float *x_scales,
                               void *Y, int M, int N, int K, int P, int nrb, int out_f32, int cus,
                               hipStream_t s) {
    const int grid = nrb < cus ? nrb : cus;
    const int T = q8_pick_t<MT>(P);
    if (MT == 1) {
        if (T == 2) q8_launch<1, 2, GROUPS>(grid, s, packed, X, x_scales, Y, M, N, K, P, nrb, out_f32);
        else q8_launch<1, 3, GROUPS>(grid, s, packed, X, x_scales, Y, M, N, K, P, nrb, out_f32);
    } else {
        if (T == 1) q8_launch<2, 1, GROUPS>(grid, s, packed, X, x_scales, Y, M, N, K, P, nrb, out_f32);
        else q8_launch<2, 2, GROUPS>(grid, s, packed, X, x_scales, Y, M, N, K, P, nrb, out_f32);
    }
    return hipGetLastError();
}

hipError_t launch_q8_skinny(const uint8_t *packed, const int8_t *X, const float *x_scales,
                            void *Y, int64_t M, int64_t N, int64_t K, int out_mode, int cus,
                            hipStream_t s) {
    const int P = (int)ceil_div(K, Q8_TILE_K);
    const int nrb = (int)ceil_div(N, RB);
    const int f32 = out_mode == 1 ? 1 : 0;
    if (out_mode == 2)
        return M <= 16 ? launch_q8_mt<1, true>(packed, X, x_scales, Y, (int)M, (int)N, (int)K, P, nrb, 0, cus, s)
                       : launch_q8_mt<2, true>(packed, X, x_scales, Y, (int)M, (int)N, (int)K, P, nrb, 0, cus, s);
    return M <= 16 ? launch_q8_mt<1, false>(packed, X, x_scales, Y, (int)M, (int)N, (int)K, P, nrb, f32, cus, s)
                   : launch_q8_mt<2, false>(packed, X, x_scales, Y, (int)M, (int)N, (int)K, P, nrb, f32, cus, s);
}

}  // namespace qg
