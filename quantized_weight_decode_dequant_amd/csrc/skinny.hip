// Skinny Q4 product Y[M, N] = X[M, K] W^T for M = 2..32 bf16 activation
// rows, single matrices too small for the streaming kernel
// (q4_skinny_stream.hip) to give each of its waves rowblocks of their own:
// every projection of a decode step except the lm_head, called one at a
// time during a verification pass (Uzu page, fange-kb.cn, section
// "Producing several tokens from one model pass": sixteen candidate rows
// give the matrix units sixteen rows of work instead of one).
//
// Arithmetic per tile as in the streaming kernel: each packed word becomes
// the bf16x8 B operand (128 + q) of one v_mfma_f32_16x16x32_bf16 (lane l: 8
// consecutive k of weight row l & 15, k-slice l >> 4), one MFMA pair covers
// one group of 64 and acc += s * C + (b - 128 s) * sum_g X.
//
// Work split.  One workgroup of 16 waves per CU holds a K-segment of X (all
// rows, 4096 k for up to 16 rows, 2048 k for up to 32; rows padded by 16
// bytes so the 16 A-operand rows of an MFMA hit distinct banks) with its
// per-(group, row) sums in LDS, and walks rowblocks in a grid-strided loop.
// Within a rowblock the 16 waves split K: wave w takes T consecutive tiles
// of each segment, so even a matrix of 256 rowblocks keeps every wave of
// every CU loading.  When K is one segment, X is staged once and the next
// rowblock's weight loads go out before the current rowblock's arithmetic.
// When K spans segments, the segments are the outer loop: a workgroup with
// several rowblocks (up to 4) stages each segment's X once for all of them,
// adds each (rowblock, segment) partial of its 16 waves into the rowblock's
// sums in LDS and loads the next rowblock's weights during the current one's
// arithmetic; a workgroup with one rowblock keeps its sums in registers.
// The 16 wave partials of a rowblock are added in wave order, the segments
// in order (deterministic).  Weight tiles past the end of K read as zero (their
// offsets sit in the range-checked part of the buffer address), and so does
// X past K and past row M, so ragged shapes need no branches.
#include <algorithm>

#include "qg_internal.h"

namespace qg {

constexpr int SK_WAVES = 16;
constexpr int SK_THREADS = SK_WAVES * 64;
constexpr int SK_RMAX = 4;  // rowblocks per workgroup when K spans several segments

template <int MT, int T>
struct SkCfg {
    static constexpr int MP = 16 * MT;               // padded activation rows
    static constexpr int SEGT = SK_WAVES * T;        // tiles per staged segment
    // LDS row stride in bf16: rows 8 dwords apart modulo the 128 banks, so the
    // 16-byte operand reads of 16 rows x 2 k-pieces hit distinct banks
    static constexpr int RS = SEGT * Q4_TILE_K + 16;
    static constexpr size_t LDS_X = (size_t)MP * RS * 2;
    static constexpr size_t LDS_XS = (size_t)2 * SEGT * MP * 4;
    static constexpr size_t LDS_RED = (size_t)SK_WAVES * 64 * 16;
    // the workgroup's rowblock sums across segments: [SK_RMAX][MT][64] f32x4
    static constexpr size_t LDS_ACC = (size_t)SK_RMAX * MT * 64 * 16;
    static_assert(LDS_X + LDS_XS + LDS_RED + LDS_ACC <= 160 * 1024, "LDS budget");
};

template <int T>
struct SkW {
    u32x4_t c[T];
    u32x2_t sb[T];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sk_rsrc(const uint8_t *packed, int rb, int P,
                                                          bool valid) {
    const unsigned bytes = (unsigned)P * Q4_TILE_BYTES;
    return make_rsrc(uniform_ptr(packed + (size_t)rb * bytes), valid ? bytes : 0u);
}

// The loads of tiles [p0, p0 + T) of one rowblock (buffer rw over its P
// tiles; an empty buffer, or tiles past P, read as zero).
template <int T>
__device__ __forceinline__ void sk_load(SkW<T> &B, __amdgpu_buffer_rsrc_t rw, int p0, int lane) {
    const unsigned lc = 16u * lane, ls = 1024u + 8u * (lane & 15);
#pragma unroll
    for (int j = 0; j < T; ++j) {
        const unsigned tw = (unsigned)(p0 + j) * Q4_TILE_BYTES;
        B.c[j] = buf_ld_x4(rw, tw + lc, 0);
        B.sb[j] = buf_ld_x2(rw, tw + ls, 0);
    }
}

// Stage segment `seg` of X (SEGT tiles; zero past K and past row M) and the
// sums of each row over each group of 64: xs[g * MP + m].
template <int MT, int T>
__device__ __forceinline__ void sk_stage(const uint16_t *X, int M, int K, int seg, uint16_t *xl,
                                         float *xs, int tid) {
    typedef SkCfg<MT, T> C;
    const int k0 = seg * C::SEGT * Q4_TILE_K;
    constexpr int PER_ROW = C::SEGT * 16;  // 16-byte chunks per row
    constexpr int TOTAL = C::MP * PER_ROW;
    constexpr int U = 4;
#pragma unroll 1
    for (int i0 = tid; i0 < TOTAL; i0 += U * SK_THREADS) {
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * SK_THREADS;
            const int m = i / PER_ROW, c8 = i - m * PER_ROW;
            const int k = k0 + 8 * c8;
            v[u] = (i < TOTAL && m < M && k < K)
                       ? ld_global(reinterpret_cast<const u32x4_t *>(X + (size_t)m * K + k))
                       : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * SK_THREADS;
            const int m = i / PER_ROW, c8 = i - m * PER_ROW;
            if (i < TOTAL) *reinterpret_cast<u32x4_t *>(xl + m * C::RS + 8 * c8) = v[u];
        }
    }
    __syncthreads();
    for (int i = tid; i < 2 * C::SEGT * C::MP; i += SK_THREADS) {
        const int g = i / C::MP, m = i - g * C::MP;
        const uint4 *rr = reinterpret_cast<const uint4 *>(xl + m * C::RS + g * 64);
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
}

// This wave's T tiles (segment-relative index ps of the first) into acc.
template <int MT, int T>
__device__ __forceinline__ void sk_compute(const SkW<T> &B, const uint16_t *xl, const float *xs,
                                           int ps, int lane, const Q4Consts &kq,
                                           f32x4_t acc[MT]) {
    typedef SkCfg<MT, T> C;
    const int kg = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int j = 0; j < T; ++j) {
        // one tile's operands live at a time
        __builtin_amdgcn_sched_barrier(0);
        bf16x8_t Bq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) Bq[q] = q4_word_to_bf16x8(B.c[j][q], kq);
        const float s0 = f16_lo(B.sb[j][0]), b0 = f16_hi(B.sb[j][0]);
        const float s1 = f16_lo(B.sb[j][1]), b1 = f16_hi(B.sb[j][1]);
        const float bb0 = fmaf(-128.f, s0, b0), bb1 = fmaf(-128.f, s1, b1);
        const int p = ps + j;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint16_t *ar = xl + (16 * mt + r16) * C::RS + p * Q4_TILE_K + 8 * kg;
            bf16x8_t A[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) A[q] = *reinterpret_cast<const bf16x8_t *>(ar + 32 * q);
            const f32x4_t xs0 = *reinterpret_cast<const f32x4_t *>(xs + (2 * p) * C::MP + 16 * mt + 4 * kg);
            const f32x4_t xs1 = *reinterpret_cast<const f32x4_t *>(xs + (2 * p + 1) * C::MP + 16 * mt + 4 * kg);
            f32x4_t C0 = {0.f, 0.f, 0.f, 0.f}, C1 = {0.f, 0.f, 0.f, 0.f};
            C0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], Bq[0], C0, 0, 0, 0);
            C0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1], Bq[1], C0, 0, 0, 0);
            C1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[2], Bq[2], C1, 0, 0, 0);
            C1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[3], Bq[3], C1, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float a = acc[mt][e];
                a = fmaf(s0, C0[e], a);
                a = fmaf(bb0, xs0[e], a);
                a = fmaf(s1, C1[e], a);
                a = fmaf(bb1, xs1[e], a);
                acc[mt][e] = a;
            }
        }
    }
}

// Sum the 16 waves' partials of rowblock rb in wave order; wave 0 writes Y.
template <int MT>
__device__ __forceinline__ void sk_finish(const f32x4_t acc[MT], f32x4_t (*red)[64], int wave,
                                          int lane, int rb, int M, const WorkItem &it) {
    const int kg = lane >> 4, n = rb * RB + (lane & 15);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        red[wave][lane] = acc[mt];
        __syncthreads();
        if (wave == 0) {
            f32x4_t s = red[0][lane];
#pragma unroll
            for (int w = 1; w < SK_WAVES; ++w) s += red[w][lane];
            if (n < it.N) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = 16 * mt + 4 * kg + e;
                    if (m < M) {
                        if (it.out_f32)
                            st_global<float>(it.y, (size_t)m * it.N + n, s[e]);
                        else
                            st_global<uint16_t>(it.y, (size_t)m * it.N + n, f32_to_bf16(s[e]));
                    }
                }
            }
        }
        __syncthreads();
    }
}

// Add this segment's partials of a rowblock (the 16 waves' acc, in wave
// order) to the rowblock's sums in LDS (set on the first segment): segments
// are added in order, so the result is deterministic.
template <int MT>
__device__ __forceinline__ void sk_accumulate(const f32x4_t acc[MT], f32x4_t (*red)[64],
                                              f32x4_t *accl, bool first, int wave, int lane) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        red[wave][lane] = acc[mt];
        __syncthreads();
        if (wave == mt) {
            f32x4_t s = red[0][lane];
#pragma unroll
            for (int w = 1; w < SK_WAVES; ++w) s += red[w][lane];
            accl[mt * 64 + lane] = first ? s : accl[mt * 64 + lane] + s;
        }
        __syncthreads();
    }
}

// Write a rowblock's sums from LDS (wave mt writes m-tile mt).
template <int MT>
__device__ __forceinline__ void sk_write(const f32x4_t *accl, int wave, int lane, int rb, int M,
                                         const WorkItem &it) {
    if (wave >= MT) return;
    const int kg = lane >> 4, n = rb * RB + (lane & 15);
    if (n >= it.N) return;
    const f32x4_t s = accl[wave * 64 + lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int m = 16 * wave + 4 * kg + e;
        if (m < M) {
            if (it.out_f32)
                st_global<float>(it.y, (size_t)m * it.N + n, s[e]);
            else
                st_global<uint16_t>(it.y, (size_t)m * it.N + n, f32_to_bf16(s[e]));
        }
    }
}

template <int MT>
__device__ __forceinline__ void sk_zero(f32x4_t a[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) a[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

template <int MT, int T>
__global__ void __launch_bounds__(SK_THREADS, 1)
q4_skinny_kernel(WorkItem it, int M) {
    typedef SkCfg<MT, T> C;
    __shared__ __attribute__((aligned(16))) uint16_t xl[C::MP * C::RS];
    __shared__ __attribute__((aligned(16))) float xs[2 * C::SEGT * C::MP];
    __shared__ f32x4_t red[SK_WAVES][64];
    __shared__ f32x4_t accl[SK_RMAX * MT * 64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Q4Consts kq = q4_consts();
    const uint16_t *X = reinterpret_cast<const uint16_t *>(it.x);
    const int P = it.P, nrb = it.units;
    const int nseg = (P + C::SEGT - 1) / C::SEGT;
    int rb = blockIdx.x;
    if (rb >= nrb) return;
    f32x4_t acc[MT];
    SkW<T> A, B;
    if (nseg == 1) {
        // X staged once; the next rowblock's weights load during this one's
        // arithmetic
        const int p0 = wave * T;
        sk_load<T>(A, sk_rsrc(it.packed, rb, P, true), p0, lane);
        sk_stage<MT, T>(X, M, it.K, 0, xl, xs, tid);
#pragma unroll 1
        for (;;) {
            int nx = rb + gridDim.x;
            sk_load<T>(B, sk_rsrc(it.packed, nx, P, nx < nrb), p0, lane);
            __builtin_amdgcn_sched_barrier(0);
            sk_zero<MT>(acc);
            sk_compute<MT, T>(A, xl, xs, p0, lane, kq, acc);
            sk_finish<MT>(acc, red, wave, lane, rb, M, it);
            if (nx >= nrb) break;
            rb = nx;
            nx = rb + gridDim.x;
            sk_load<T>(A, sk_rsrc(it.packed, nx, P, nx < nrb), p0, lane);
            __builtin_amdgcn_sched_barrier(0);
            sk_zero<MT>(acc);
            sk_compute<MT, T>(B, xl, xs, p0, lane, kq, acc);
            sk_finish<MT>(acc, red, wave, lane, rb, M, it);
            if (nx >= nrb) break;
            rb = nx;
        }
        return;
    }
    // several segments per rowblock: segments outermost.  The workgroup's
    // rowblocks (at most SK_RMAX, grid-strided) keep their sums in LDS across
    // the segments, so X is staged once per segment; the weights of the next
    // (rowblock, segment) load during the current one's arithmetic, and the
    // first rowblock's weights of a segment before its X is staged.
    const int rpw = (nrb - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    if (rpw == 1) {
        // one rowblock: its sums stay in registers across the segments, each
        // segment's weight loads issued before its X is staged
        sk_zero<MT>(acc);
#pragma unroll 1
        for (int seg = 0; seg < nseg; ++seg) {
            sk_load<T>(A, sk_rsrc(it.packed, rb, P, true), seg * C::SEGT + wave * T, lane);
            __syncthreads();  // nobody still reads the previous segment
            sk_stage<MT, T>(X, M, it.K, seg, xl, xs, tid);
            sk_compute<MT, T>(A, xl, xs, wave * T, lane, kq, acc);
        }
        sk_finish<MT>(acc, red, wave, lane, rb, M, it);
        return;
    }
    sk_load<T>(A, sk_rsrc(it.packed, rb, P, true), wave * T, lane);
#pragma unroll 1
    for (int seg = 0; seg < nseg; ++seg) {
        __syncthreads();  // nobody still reads the previous segment
        sk_stage<MT, T>(X, M, it.K, seg, xl, xs, tid);
        const int p0 = seg * C::SEGT + wave * T;
        const bool nseg_next = seg + 1 < nseg;
#pragma unroll 1
        for (int i = 0; i < rpw; i += 2) {
            // rowblock i from A while the next (rowblock i + 1, or the first
            // of the next segment) loads into B
            {
                const bool more = i + 1 < rpw;
                sk_load<T>(B, sk_rsrc(it.packed, more ? rb + (i + 1) * (int)gridDim.x : rb, P,
                                      more || nseg_next),
                           more ? p0 : p0 + C::SEGT, lane);
                __builtin_amdgcn_sched_barrier(0);
                sk_zero<MT>(acc);
                sk_compute<MT, T>(A, xl, xs, wave * T, lane, kq, acc);
                sk_accumulate<MT>(acc, red, accl + i * MT * 64, seg == 0, wave, lane);
                if (!more) {
                    // the next segment starts from A
#pragma unroll
                    for (int j = 0; j < T; ++j) {
                        A.c[j] = B.c[j];
                        A.sb[j] = B.sb[j];
                    }
                    break;
                }
            }
            // rowblock i + 1 from B while the next loads into A
            {
                const bool more = i + 2 < rpw;
                sk_load<T>(A, sk_rsrc(it.packed, more ? rb + (i + 2) * (int)gridDim.x : rb, P,
                                      more || nseg_next),
                           more ? p0 : p0 + C::SEGT, lane);
                __builtin_amdgcn_sched_barrier(0);
                sk_zero<MT>(acc);
                sk_compute<MT, T>(B, xl, xs, wave * T, lane, kq, acc);
                sk_accumulate<MT>(acc, red, accl + (i + 1) * MT * 64, seg == 0, wave, lane);
            }
        }
    }
#pragma unroll 1
    for (int i = 0; i < rpw; ++i)
        sk_write<MT>(accl + i * MT * 64, wave, lane, rb + i * (int)gridDim.x, M, it);
}

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
    const int segt = M <= 16 ? (it.P <= SkCfg<1, 1>::SEGT ? SkCfg<1, 1>::SEGT : SkCfg<1, 2>::SEGT)
                             : SkCfg<2, 1>::SEGT;
    // one workgroup per CU (fewer CUs for fewer rowblocks), and when K spans
    // segments at most SK_RMAX rowblocks per workgroup
    int grid = it.units < cus ? it.units : cus;
    if (it.P > segt) grid = (int)std::max<int64_t>(ceil_div(it.units, SK_RMAX), grid);
    if (M <= 16) {
        // 2 tiles per wave (4096 k per segment) unless one tile per wave
        // already covers K in one segment
        if (it.P <= SkCfg<1, 1>::SEGT)
            hipLaunchKernelGGL((q4_skinny_kernel<1, 1>), dim3(grid), dim3(SK_THREADS), 0, s, it, (int)M);
        else
            hipLaunchKernelGGL((q4_skinny_kernel<1, 2>), dim3(grid), dim3(SK_THREADS), 0, s, it, (int)M);
    } else {
        hipLaunchKernelGGL((q4_skinny_kernel<2, 1>), dim3(grid), dim3(SK_THREADS), 0, s, it, (int)M);
    }
    return hipGetLastError();
}

}  // namespace qg
