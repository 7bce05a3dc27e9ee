// Skinny product Y[M, N] = X[M, K] W^T, M = 2..32 bf16 activation rows, for
// the affine weight family ("MLX Runner: An Inference Engine You Can Read",
// section "Architecture: one command buffer per token"): the verification
// form of a draft of several tokens (Uzu page, fange-kb.cn, section
// "Producing several tokens from one model pass": one weight read serves all
// the candidate rows).
//
// Each run of 8 codes of a lane (k = 32i + 8(lane >> 4) .. +8 of the tile)
// becomes, as pairs 128 + q, the bf16x8 B operand of one
// v_mfma_f32_16x16x32_bf16 step; the 64 lanes' runs i make up the 32-k block
// i, so a step stays inside one group, and after the steps of a group
//     acc += scale * C + (bias - 128 scale) * sum_{k in group} X[m][k]
// (8-bit codes: C = C_lo + 16 C_hi and 128 * 17 for the offset).
//
// Work split.  One workgroup per CU (16 waves; 8 for more than 16 rows)
// holds a K-segment of X (4096 k for 16 rows, 2048 k for 32) in LDS with the
// per-(group, row) sums of X.  Each wave owns every 16th (8th) rowblock of the
// workgroup's contiguous range and streams its tiles in batches,
// double-buffered across rowblocks; it keeps the sums of 4 rowblocks across
// the segments and stores them together.  When K is one segment, X is
// staged once for the whole range.  Every rowblock adds its tiles in K order
// within one wave (deterministic).
#include "affine_tile.h"

namespace qg {

template <int MT>
struct AsCfg {
    static constexpr int WAVES = MT == 1 ? 16 : 8;
    static constexpr int THREADS = WAVES * 64;
    static constexpr int MP = 16 * MT;                // padded activation rows
    static constexpr int SEGK = 32 / MT;              // tiles per staged segment
    // LDS row stride in bf16: rows 8 dwords apart modulo the 128 banks, so the
    // 16-byte operand reads of 16 rows x 2 k-pieces hit distinct banks
    static constexpr int RS = SEGK * AFF_TILE_K + 16;
    static constexpr int R = 4;                       // rowblocks kept across segments
    static constexpr size_t LDS_X = (size_t)MP * RS * 2;
    // group sums: at most SEGK * 4 groups (group 32) per segment
    static constexpr size_t LDS = LDS_X + (size_t)SEGK * 4 * MP * 4;
};
static_assert(AsCfg<1>::LDS <= 160 * 1024 && AsCfg<2>::LDS <= 160 * 1024, "LDS budget");

// tiles per batch: 2, or 1 when a lane's words of a tile are many (larger
// batches keep too many operands live and spill)
template <int BITS, int GPT>
struct AsBatchSize {
    typedef AffPlanes<BITS> PL;
    static constexpr int WORDS = PL::W0 + (PL::NP == 2 ? PL::W1 : 0) + GPT;
    static constexpr int TPB = WORDS <= 8 ? 2 : 1;
};

template <int BITS, int GPT>
struct AsBatch {
    AgTile<BITS, GPT> t[AsBatchSize<BITS, GPT>::TPB];
};

// Stage tiles [0, nt) of segment seg of X (rows past M and k past K zero) and
// the sum of each row over each group: xs[gi * MP + m].
constexpr int AS_SU = 8;  // staging chunks per thread in flight

template <int MT>
__device__ __forceinline__ void as_stage(const uint16_t *X, int M, int K, int seg, int nt,
                                         int group, uint16_t *xl, float *xs, int tid) {
    typedef AsCfg<MT> C;
    const int k0 = seg * C::SEGK * AFF_TILE_K;
    const int per_row = nt * (AFF_TILE_K / 8);  // 16-byte chunks per row
    const int total = C::MP * per_row;
    // each thread issues the loads of AS_SU chunks before it writes any of
    // them; buffer loads, so a chunk past the rows or past K reads zero
    const unsigned xbytes = (unsigned)M * (unsigned)K * 2u;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, xbytes);
    for (int i0 = tid; i0 < total; i0 += AS_SU * C::THREADS) {
        u32x4_t v[AS_SU];
#pragma unroll
        for (int u = 0; u < AS_SU; ++u) {
            const int i = i0 + u * C::THREADS, m = i / per_row, c8 = i - m * per_row;
            const int k = k0 + 8 * c8;
            const unsigned off =
                (m < M && k < K) ? 2u * ((unsigned)m * (unsigned)K + (unsigned)k) : xbytes;
            v[u] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0));
        }
#pragma unroll
        for (int u = 0; u < AS_SU; ++u) {
            const int i = i0 + u * C::THREADS, m = i / per_row, c8 = i - m * per_row;
            if (i < total) *reinterpret_cast<u32x4_t *>(xl + m * C::RS + 8 * c8) = v[u];
        }
    }
    __syncthreads();
    const int ng = nt * (AFF_TILE_K / group);
    for (int i = tid; i < ng * C::MP; i += C::THREADS) {
        const int gi = i / C::MP, m = i - gi * C::MP;
        const uint4 *rr = reinterpret_cast<const uint4 *>(xl + m * C::RS + gi * group);
        float sum = 0.f;
        for (int q = 0; q < group / 8; ++q) {
            const uint4 w = rr[q];
            sum += ((bf16_lo(w.x) + bf16_hi(w.x)) + (bf16_lo(w.y) + bf16_hi(w.y))) +
                   ((bf16_lo(w.z) + bf16_hi(w.z)) + (bf16_lo(w.w) + bf16_hi(w.w)));
        }
        xs[i] = sum;
    }
    __syncthreads();
}

// One tile (index pl within the staged segment) into acc.
template <int BITS, int GPT, int MT, bool BF16S>
__device__ __forceinline__ void as_tile(const AgTile<BITS, GPT> &T, const uint16_t *xl,
                                        const float *xs, int pl, int lane, f32x4_t acc[MT],
                                        const AgConsts &k) {
    typedef AsCfg<MT> C;
    constexpr int CPG = 4 / GPT;  // MFMA steps (32-k blocks) per group
    const int kg = lane >> 4, r16 = lane & 15;
    const f32x4_t Z = {0.f, 0.f, 0.f, 0.f};
    f32x4_t Cl[MT], Ch[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) Cl[mt] = Ch[mt] = Z;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4_t bl = {ag_bf16_pair<BITS, GPT>(T, 4 * i, k),
                            ag_bf16_pair<BITS, GPT>(T, 4 * i + 1, k),
                            ag_bf16_pair<BITS, GPT>(T, 4 * i + 2, k),
                            ag_bf16_pair<BITS, GPT>(T, 4 * i + 3, k)};
        u32x4_t bh = {0u, 0u, 0u, 0u};
        if constexpr (BITS == 8)
            bh = u32x4_t{ag_pair_hi<BITS, GPT>(T, 4 * i, k), ag_pair_hi<BITS, GPT>(T, 4 * i + 1, k),
                         ag_pair_hi<BITS, GPT>(T, 4 * i + 2, k),
                         ag_pair_hi<BITS, GPT>(T, 4 * i + 3, k)};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const bf16x8_t A = *reinterpret_cast<const bf16x8_t *>(
                xl + (16 * mt + r16) * C::RS + pl * AFF_TILE_K + 32 * i + 8 * kg);
            Cl[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8_t, bl),
                                                            Cl[mt], 0, 0, 0);
            if constexpr (BITS == 8)
                Ch[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    A, __builtin_bit_cast(bf16x8_t, bh), Ch[mt], 0, 0, 0);
        }
        if ((i + 1) % CPG == 0) {
            const int t = i / CPG;
            const unsigned sb = T.sb[t];
            const float s = ag_scale(sb, BF16S), b = ag_bias(sb, BF16S);
            const float bb = fmaf(BITS == 8 ? -2176.f : -128.f, s, b);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const f32x4_t xsv = *reinterpret_cast<const f32x4_t *>(
                    xs + (pl * GPT + t) * C::MP + 16 * mt + 4 * kg);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = BITS == 8 ? fmaf(16.f, Ch[mt][e], Cl[mt][e]) : Cl[mt][e];
                    acc[mt][e] = fmaf(s, v, fmaf(bb, xsv[e], acc[mt][e]));
                }
                Cl[mt] = Z;
                Ch[mt] = Z;
            }
        }
    }
}

template <int MT>
__device__ __forceinline__ void as_store(void *Y, bool out_f32, int N, int M, int rb,
                                         const f32x4_t acc[MT], int lane) {
    const int n = rb * RB + (lane & 15), kg = lane >> 4;
    if (n >= N) return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 16 * mt + 4 * kg + e;
            if (m < M) {
                if (out_f32)
                    st_global<float>(Y, (size_t)m * N + n, acc[mt][e]);
                else
                    st_global<uint16_t>(Y, (size_t)m * N + n, f32_to_bf16(acc[mt][e]));
            }
        }
}

// This wave's rowblocks i0 .. i0 + n - 1 (wave rowblock i is first + WAVES i)
// over one segment (tiles pbase .. pbase + pn), each into acc[r] (r a
// compile-time index).  A rowblock's batches are rounded up to an even count
// so that the double buffer alternates identically for every rowblock (a
// padding batch reads through an empty buffer and meets zero X, adding
// exactly zero); its last batch step loads the next rowblock's first batch.
// A holds the block's first batch on entry.
template <int BITS, int GPT, int MT, bool BF16S>
__device__ __forceinline__ void as_block(AsBatch<BITS, GPT> &A, AsBatch<BITS, GPT> &B,
                                         const uint8_t *packed, size_t rb_bytes, unsigned tb,
                                         int first, int i0, int n, int pbase, int pn,
                                         const uint16_t *xl, const float *xs, int lane,
                                         f32x4_t acc[AsCfg<MT>::R][MT], const AgConsts &k) {
    typedef AsCfg<MT> C;
    constexpr int TPB = AsBatchSize<BITS, GPT>::TPB;
    const int nbs = (pn + TPB - 1) / TPB, nbe = nbs + (nbs & 1);
#pragma unroll
    for (int r = 0; r < C::R; ++r) {
        if (r >= n) break;  // uniform
        const int rb = first + C::WAVES * (i0 + r), rbn = rb + C::WAVES;
        const bool vnext = r + 1 < n;
        const uint8_t *base = packed + (size_t)rb * rb_bytes + (size_t)pbase * tb;
        const uint8_t *basen = packed + (size_t)rbn * rb_bytes + (size_t)pbase * tb;
#pragma unroll 1
        for (int bt = 0; bt < nbe; bt += 2) {
            // batch bt (in A) computed while bt + 1 loads into B
            {
                const __amdgpu_buffer_rsrc_t rs =
                    make_rsrc(uniform_ptr(base), bt + 1 < nbs ? (unsigned)pn * tb : 0u);
#pragma unroll
                for (int q = 0; q < TPB; ++q) {
                    __builtin_amdgcn_sched_barrier(0);
                    ag_tile_load<BITS, GPT>(B.t[q], rs, (bt + 1) * TPB + q, pn, tb, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    as_tile<BITS, GPT, MT, BF16S>(A.t[q], xl, xs, bt * TPB + q, lane, acc[r], k);
                }
            }
            // batch bt + 1 (in B) computed while bt + 2, or the next
            // rowblock's first batch, loads into A
            {
                const bool more = bt + 2 < nbe;
                const __amdgpu_buffer_rsrc_t rs =
                    more ? make_rsrc(uniform_ptr(base), bt + 2 < nbs ? (unsigned)pn * tb : 0u)
                         : make_rsrc(uniform_ptr(vnext ? basen : base), vnext ? (unsigned)pn * tb : 0u);
                const int tn = more ? (bt + 2) * TPB : 0;
#pragma unroll
                for (int q = 0; q < TPB; ++q) {
                    __builtin_amdgcn_sched_barrier(0);
                    ag_tile_load<BITS, GPT>(A.t[q], rs, tn + q, pn, tb, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    as_tile<BITS, GPT, MT, BF16S>(B.t[q], xl, xs, (bt + 1) * TPB + q, lane, acc[r], k);
                }
            }
        }
    }
}

// The first batch of rowblock rb over one segment.
template <int BITS, int GPT>
__device__ __forceinline__ void as_first(AsBatch<BITS, GPT> &A, const uint8_t *packed,
                                         size_t rb_bytes, unsigned tb, int rb, int pbase, int pn,
                                         bool valid, int lane) {
    constexpr int TPB = AsBatchSize<BITS, GPT>::TPB;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(uniform_ptr(packed + (size_t)rb * rb_bytes + (size_t)pbase * tb),
                  valid ? (unsigned)pn * tb : 0u);
#pragma unroll
    for (int q = 0; q < TPB; ++q) ag_tile_load<BITS, GPT>(A.t[q], rs, q, pn, tb, lane);
}

// Rowblocks [u0, u1) of one matrix: wave w owns rowblocks u0 + w + WAVES i;
// X staged per segment (once for the range when K is one segment).
template <int BITS, int GPT, int MT, bool BF16S>
__device__ __forceinline__ void as_range(const WorkItem &it, int u0, int u1, int M, uint16_t *xl,
                                         float *xs, int tid, int lane, int wave,
                                         const AgConsts &kc) {
    typedef AsCfg<MT> C;
    constexpr int R = C::R;
    constexpr int TPB = AsBatchSize<BITS, GPT>::TPB;
    const int group = AFF_TILE_K / GPT;
    const unsigned tb = (unsigned)affine_tile_bytes(BITS, group);
    const int P = it.P;
    const size_t rb_bytes = (size_t)P * tb;
    const uint8_t *packed = it.packed;
    const uint16_t *X = reinterpret_cast<const uint16_t *>(it.x);
    const int nseg = (P + C::SEGK - 1) / C::SEGK;
    const int first = u0 + wave;
    const int mine = (u1 - u0 > wave) ? (u1 - u0 - wave + C::WAVES - 1) / C::WAVES : 0;
    const int slots = (u1 - u0 + C::WAVES - 1) / C::WAVES;  // wave 0 has the most
    AsBatch<BITS, GPT> A, B;
    f32x4_t acc[R][MT];
#pragma unroll 1
    for (int i0 = 0; i0 < slots; i0 += R) {
        const int n = max(0, min(R, mine - i0));
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[r][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int seg = 0; seg < nseg; ++seg) {
            const int pbase = seg * C::SEGK, pn = min(C::SEGK, P - pbase);
            const int nbs = (pn + TPB - 1) / TPB, nbe = nbs + (nbs & 1);
            as_first<BITS, GPT>(A, packed, rb_bytes, tb, first + C::WAVES * i0, pbase, pn, n > 0,
                                lane);
            if (nseg > 1 || i0 == 0) {
                __syncthreads();  // nobody still reads the previous segment of X
                as_stage<MT>(X, M, it.K, seg, nbe * TPB, group, xl, xs, tid);
            }
            if (n > 0)
                as_block<BITS, GPT, MT, BF16S>(A, B, packed, rb_bytes, tb, first, i0, n, pbase, pn,
                                               xl, xs, lane, acc, kc);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (r < n)
                as_store<MT>(it.y, it.out_f32 != 0, it.N, M, first + C::WAVES * (i0 + r), acc[r],
                             lane);
    }
}

// LIST = false: one matrix (`single`, workgroup j takes rowblocks
// [j n / G, (j + 1) n / G)); LIST = true: the work list (workgroup j walks
// the (matrix, rowblock) range [starts[j], starts[j + 1])).  Work index j is
// XCD-aware, so consecutive ranges share an L2.
template <bool LIST, int BITS, int GPT, int MT, bool BF16S>
__global__ void __launch_bounds__(AsCfg<MT>::THREADS, 1)
affine_skinny_kernel(const WorkItem *__restrict__ items, const WorkStart *__restrict__ starts,
                     WorkItem single, int M) {
    typedef AsCfg<MT> C;
    __shared__ __attribute__((aligned(16))) uint16_t xl[C::MP * C::RS];
    __shared__ __attribute__((aligned(16))) float xs[C::SEGK * 4 * C::MP];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const AgConsts kc = ag_consts<BITS>();
    const int wg = xcd_work_index(blockIdx.x, gridDim.x);
    if (!LIST) {
        const int64_t G = gridDim.x, n = single.units;
        const int u0 = (int)(wg * n / G), u1 = (int)((wg + 1) * n / G);
        if (u0 < u1) as_range<BITS, GPT, MT, BF16S>(single, u0, u1, M, xl, xs, tid, lane, wave, kc);
        return;
    }
    const WorkStart s = starts[wg], e = starts[wg + 1];
#pragma unroll 1
    for (int i = s.item; i < e.item || (i == e.item && e.unit > 0); ++i) {
        const WorkItem it = items[i];
        const int u0 = (i == s.item) ? s.unit : 0;
        const int u1 = (i == e.item) ? e.unit : it.units;
        if (u0 < u1) as_range<BITS, GPT, MT, BF16S>(it, u0, u1, M, xl, xs, tid, lane, wave, kc);
    }
}

template <bool LIST, int BITS, int GPT, int MT, bool BF16S>
static void launch_as1(const WorkItem *items, const WorkStart *starts, const WorkItem &it, int M,
                       int grid, hipStream_t s) {
    hipLaunchKernelGGL((affine_skinny_kernel<LIST, BITS, GPT, MT, BF16S>), dim3(grid),
                       dim3(AsCfg<MT>::THREADS), 0, s, items, starts, it, M);
}

template <bool LIST, int BITS, int GPT>
static hipError_t launch_as(const WorkItem *items, const WorkStart *starts, const WorkItem &it,
                            int64_t M, bool bf16, int grid, hipStream_t s) {
    if (M <= 16) {
        if (bf16)
            launch_as1<LIST, BITS, GPT, 1, true>(items, starts, it, (int)M, grid, s);
        else
            launch_as1<LIST, BITS, GPT, 1, false>(items, starts, it, (int)M, grid, s);
    } else {
        if (bf16)
            launch_as1<LIST, BITS, GPT, 2, true>(items, starts, it, (int)M, grid, s);
        else
            launch_as1<LIST, BITS, GPT, 2, false>(items, starts, it, (int)M, grid, s);
    }
    return hipGetLastError();
}

template <bool LIST, int BITS>
static hipError_t launch_as_bits(const WorkItem *items, const WorkStart *starts,
                                 const WorkItem &it, int64_t M, int group, bool bf16, int grid,
                                 hipStream_t s) {
    switch (group) {
    case 32: return launch_as<LIST, BITS, 4>(items, starts, it, M, bf16, grid, s);
    case 64: return launch_as<LIST, BITS, 2>(items, starts, it, M, bf16, grid, s);
    default: return launch_as<LIST, BITS, 1>(items, starts, it, M, bf16, grid, s);
    }
}

template <bool LIST>
static hipError_t launch_as_fmt(const WorkItem *items, const WorkStart *starts,
                                const WorkItem &it, int bits, int group, bool bf16, int64_t M,
                                int grid, hipStream_t s) {
    switch (bits) {
    case 2: return launch_as_bits<LIST, 2>(items, starts, it, M, group, bf16, grid, s);
    case 3: return launch_as_bits<LIST, 3>(items, starts, it, M, group, bf16, grid, s);
    case 4: return launch_as_bits<LIST, 4>(items, starts, it, M, group, bf16, grid, s);
    case 5: return launch_as_bits<LIST, 5>(items, starts, it, M, group, bf16, grid, s);
    case 6: return launch_as_bits<LIST, 6>(items, starts, it, M, group, bf16, grid, s);
    case 8: return launch_as_bits<LIST, 8>(items, starts, it, M, group, bf16, grid, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_affine_skinny(const uint8_t *packed, const uint16_t *X, void *Y, int bits,
                                int group, bool bf16_scales, int64_t M, int64_t N, int64_t K,
                                bool out_f32, int cus, hipStream_t s) {
    WorkItem it{};
    it.packed = packed;
    it.x = X;
    it.y = Y;
    it.N = (int32_t)N;
    it.K = (int32_t)K;
    it.P = (int32_t)ceil_div(K, AFF_TILE_K);
    it.units = (int32_t)ceil_div(N, RB);
    it.out_f32 = out_f32 ? 1 : 0;
    const int grid = it.units < cus ? it.units : cus;
    return launch_as_fmt<false>(nullptr, nullptr, it, bits, group, bf16_scales, M, grid, s);
}

int affine_skinny_wgs_per_cu() { return 1; }

hipError_t launch_affine_skinny_list(const WorkItem *items, const WorkStart *starts, int grid,
                                     int bits, int group, bool bf16_scales, int64_t M,
                                     hipStream_t s) {
    WorkItem none{};
    return launch_as_fmt<true>(items, starts, none, bits, group, bf16_scales, M, grid, s);
}

}  // namespace qg
