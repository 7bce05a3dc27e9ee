// Streaming skinny Q4 product Y[M, N] = X[M, K] W^T, M = 2..32 bf16
// activation rows, for passes that stream many rowblocks per workgroup: the
// grouped verification pass over every projection of a decode step and
// single matrices with thousands of rowblocks (Uzu page, fange-kb.cn, section
// "Producing several tokens from one model pass": one weight read serves all
// the candidate rows).  Arithmetic per tile as in skinny.hip: each packed word
// becomes the bf16x8 MFMA operand (128 + q); one v_mfma_f32_16x16x32_bf16
// pair covers one group of 64 and acc += s * C + (b - 128 s) * sum_g X.
//
// Work split.  One workgroup per CU (16 waves; 8 for 32 rows) holds a
// whole 4096-k slice of X (16 rows; 2048 k for 32 rows) in LDS, 128 KB, with
// the per-(group, row) sums of X, so X is staged once per matrix and
// segment.  Each wave owns every 16th (8th) rowblock of the workgroup's
// range and streams its batches (4 consecutive 128-k tiles of one rowblock;
// at 32 rows 2 tiles of each of two rowblocks, see pair mode) double-
// buffered: the load of each tile of the next batch is issued just before
// the arithmetic of the same tile of the current batch.  The 16 x M results
// of 6 rowblocks (8 at 32 rows) stay in the wave's registers and are stored together; when
// K spans several segments those are the rowblocks whose sums the wave
// keeps across the segments.  Every rowblock accumulates its
// tiles in K order within one wave, so single and grouped launches give
// identical results.  Tiles past the end of K re-read the
// last tile; X and its sums are staged as zero there, so they add exactly
// zero.
#include "qg_internal.h"

namespace qg {

constexpr int SS_TPB = 4;  // tiles per batch

template <int MT>
struct SsCfg {
    // waves per workgroup: the most whose registers fit without real spills
    static constexpr int WAVES = MT == 1 ? 16 : 8;
    static constexpr int THREADS = WAVES * 64;
    // rowblocks whose results a wave keeps in registers (stored together)
    static constexpr int R = MT == 1 ? 6 : 8;
    // two rowblocks per wave at a time (see pair mode below)
    static constexpr bool PAIR = MT == 2;
    static constexpr int MP = 16 * MT;               // padded activation rows
    static constexpr int SEGK = 32 / MT;             // tiles per staged segment
    // LDS row stride in bf16: rows 8 dwords apart modulo the 128 banks, so the
    // 16-byte operand reads of 16 rows x 2 k-pieces hit distinct banks
    static constexpr int RS = SEGK * 128 + 16;
    static constexpr size_t LDS_X = (size_t)MP * RS * 2;
    static constexpr size_t LDS = LDS_X + (size_t)2 * SEGK * MP * 4;
};
static_assert(SsCfg<1>::LDS <= 160 * 1024 && SsCfg<2>::LDS <= 160 * 1024, "LDS budget");
static_assert(SsCfg<1>::SEGK % 8 == 0 && SsCfg<2>::SEGK % 8 == 0, "segments hold an even number of batches");

struct SsBatch {
    u32x4_t c[SS_TPB];
    u32x2_t sb[SS_TPB];
};

// Stage tiles [0, nt) of segment `seg` of X (rows past M and k past K are
// zero) and the sums of each row over each group of 64: xs[g * MP + m].
template <int MT>
__device__ __forceinline__ void ss_stage(const uint16_t *X, int M, int K, int seg, int nt,
                                         uint16_t *xl, float *xs, int tid) {
    typedef SsCfg<MT> C;
    const int k0 = seg * C::SEGK * Q4_TILE_K;
    const int per_row = nt * 16;  // 16-byte chunks per row
    const int total = C::MP * per_row;
    constexpr int U = 4;
#pragma unroll 1
    for (int i0 = tid; i0 < total; i0 += U * C::THREADS) {
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * C::THREADS;
            const int m = i / per_row, c8 = i - m * per_row;
            const int k = k0 + 8 * c8;
            v[u] = (i < total && m < M && k < K)
                       ? ld_global(reinterpret_cast<const u32x4_t *>(X + (size_t)m * K + k))
                       : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * C::THREADS;
            const int m = i / per_row, c8 = i - m * per_row;
            if (i < total) *reinterpret_cast<u32x4_t *>(xl + m * C::RS + 8 * c8) = v[u];
        }
    }
    __syncthreads();
    for (int i = tid; i < 2 * nt * C::MP; i += C::THREADS) {
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

// One tile (index pl within the staged segment): the two groups' products
// C_g = sum_k X (128 + q) on the bf16 MFMA, acc += s_g * C_g on the VALU.
template <int MT>
__device__ __forceinline__ void ss_tile(u32x4_t c, u32x2_t sb, const uint16_t *xl, int pl,
                                        int lane, const Q4Consts &kq, f32x4_t acc[MT]) {
    typedef SsCfg<MT> C;
    const int kg = lane >> 4, r16 = lane & 15;
    bf16x8_t B[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) B[q] = q4_word_to_bf16x8(c[q], kq);
    const float s0 = f16_lo(sb[0]), s1 = f16_lo(sb[1]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const uint16_t *ar = xl + (16 * mt + r16) * C::RS + pl * 128 + 8 * kg;
        bf16x8_t A[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) A[q] = *reinterpret_cast<const bf16x8_t *>(ar + 32 * q);
        f32x4_t C0 = {0.f, 0.f, 0.f, 0.f}, C1 = {0.f, 0.f, 0.f, 0.f};
        C0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], B[0], C0, 0, 0, 0);
        C0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1], B[1], C0, 0, 0, 0);
        C1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[2], B[2], C1, 0, 0, 0);
        C1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[3], B[3], C1, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[mt][e] = fmaf(s1, C1[e], fmaf(s0, C0[e], acc[mt][e]));
    }
}

// The bias terms of the two tiles pl, pl + 1 (groups 2 pl .. 2 pl + 3 of the
// segment): sum_g (b_g - 128 s_g)[n] * (sum_{k in g} X[m, k]), a product of
// rank 4, as one fp32 MFMA 16x16x4 per 16 activation rows into acc.  Lane l
// supplies the A operand element (row 16 mt + (l & 15), group 2 pl + (l >> 4))
// and the B operand element (group 2 pl + (l >> 4), output row l & 15), which
// is its own row's (scale, bias) word of tile pl + (l >> 5), group (l >> 4) & 1.
template <int MT>
__device__ __forceinline__ void ss_bias2(u32x2_t sba, u32x2_t sbb, const float *xs, int pl,
                                         int lane, f32x4_t acc[MT]) {
    typedef SsCfg<MT> C;
    const int kg = lane >> 4, r16 = lane & 15;
    const unsigned wa = (kg & 1) ? sba[1] : sba[0];
    const unsigned wb = (kg & 1) ? sbb[1] : sbb[0];
    const unsigned w = (kg & 2) ? wb : wa;
    const float bb = fmaf(-128.f, f16_lo(w), f16_hi(w));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const float a = xs[(2 * pl + kg) * C::MP + 16 * mt + r16];
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, acc[mt], 0, 0, 0);
    }
}

// Issue tile j's loads of batch N (tiles nb0 .. nb0 + 3 of the buffer rs,
// clamped to the last of pn tiles), then tile j's arithmetic of batch B
// (tiles pl0 ..), for j = 0..3; the bias terms after each pair of tiles.
template <int MT>
__device__ __forceinline__ void ss_step(SsBatch &N, __amdgpu_buffer_rsrc_t rs, int nb0, int pn,
                                        const SsBatch &B, int pl0, const uint16_t *xl,
                                        const float *xs, int lane, const Q4Consts &kq,
                                        f32x4_t cur[MT]) {
    const unsigned lc = 16u * lane, ls = 1024u + 8u * (lane & 15);
#pragma unroll
    for (int j = 0; j < SS_TPB; ++j) {
        __builtin_amdgcn_sched_barrier(0);
        const unsigned to = (unsigned)min(nb0 + j, pn - 1) * Q4_TILE_BYTES;
        N.c[j] = buf_ld_x4(rs, lc, to);
        N.sb[j] = buf_ld_x2(rs, ls, to);
        __builtin_amdgcn_sched_barrier(0);
        ss_tile<MT>(B.c[j], B.sb[j], xl, pl0 + j, lane, kq, cur);
        if (j & 1) ss_bias2<MT>(B.sb[j - 1], B.sb[j], xs, pl0 + j - 1, lane, cur);
    }
}

// Buffer over the segment's tiles of rowblock rb (empty when !valid: loads
// read zero without touching memory).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ss_rsrc(const WorkItem &it, int rb, int pbase,
                                                          int pn, bool valid) {
    const uint8_t *base = it.packed + ((size_t)rb * it.P + pbase) * Q4_TILE_BYTES;
    return make_rsrc(uniform_ptr(base), valid ? (unsigned)pn * Q4_TILE_BYTES : 0u);
}

// Store a rowblock's 16 x M results.
template <int MT>
__device__ __forceinline__ void ss_store(const WorkItem &it, int rb, int M, const f32x4_t acc[MT],
                                         int lane) {
    const int n = rb * RB + (lane & 15), kg = lane >> 4;
    if (n >= it.N) return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 16 * mt + 4 * kg + e;
            if (m < M) {
                if (it.out_f32)
                    st_global<float>(it.y, (size_t)m * it.N + n, acc[mt][e]);
                else
                    st_global<uint16_t>(it.y, (size_t)m * it.N + n, f32_to_bf16(acc[mt][e]));
            }
        }
}

template <int MT>
__device__ __forceinline__ void ss_zero(f32x4_t a[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) a[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// The first batch (tiles 0..3 of the segment) of rowblock rb.
__device__ __forceinline__ void ss_first(SsBatch &A, const WorkItem &it, int rb, int pbase, int pn,
                                         bool valid, int lane) {
    const __amdgpu_buffer_rsrc_t rs = ss_rsrc(it, rb, pbase, pn, valid);
    const unsigned lc = 16u * lane, ls = 1024u + 8u * (lane & 15);
#pragma unroll
    for (int j = 0; j < SS_TPB; ++j) {
        const unsigned to = (unsigned)min(j, pn - 1) * Q4_TILE_BYTES;
        A.c[j] = buf_ld_x4(rs, lc, to);
        A.sb[j] = buf_ld_x2(rs, ls, to);
    }
}

// Batches of one rowblock and segment: nb real ones (4 tiles each, the last
// possibly ragged), rounded up to an even count so that the double buffer
// alternates A, B, A, ... identically for every rowblock (the padding batch
// reads through an empty buffer and meets zero X, adding exactly zero).
__device__ __forceinline__ int ss_batches_even(int pn) {
    const int nb = (pn + SS_TPB - 1) / SS_TPB;
    return nb + (nb & 1);
}

// This wave's rowblocks i0 .. i0 + n - 1 (n <= R; rowblock of index i is
// first + WAVES * i) over one segment, each into acc[r] (r = i - i0, a
// compile-time index).  A holds the first batch of rowblock i0 on entry; on
// exit A holds the first batch of rowblock i0 + n, which is loaded (if
// nextvalid) during the last step, so the stream never drains.
template <int MT, int R>
__device__ __forceinline__ void ss_block(SsBatch &A, SsBatch &B, const WorkItem &it, int first,
                                         int i0, int n, bool nextvalid, int pbase, int pn,
                                         const uint16_t *xl, const float *xs, int lane,
                                         const Q4Consts &kq, f32x4_t acc[R][MT]) {
    typedef SsCfg<MT> C;
    const int nb = (pn + SS_TPB - 1) / SS_TPB, nbe = ss_batches_even(pn);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r >= n) break;  // uniform
        const int rb = first + C::WAVES * (i0 + r);
        const int rbn = rb + C::WAVES;  // the next rowblock's first batch follows this one's last
        const bool vnext = (r + 1 < n) || nextvalid;
#pragma unroll 1
        for (int b = 0; b < nbe; b += 2) {
            // batch b (in A) computed while b + 1 loads into B
            ss_step<MT>(B, ss_rsrc(it, rb, pbase, pn, b + 1 < nb), (b + 1) * SS_TPB, pn, A,
                        b * SS_TPB, xl, xs, lane, kq, acc[r]);
            // batch b + 1 (in B) computed while b + 2, or the next rowblock's
            // first batch, loads into A
            const bool more = b + 2 < nbe;
            ss_step<MT>(A, ss_rsrc(it, more ? rb : rbn, pbase, pn, more ? (b + 2 < nb) : vnext),
                        more ? (b + 2) * SS_TPB : 0, pn, B, (b + 1) * SS_TPB, xl, xs, lane, kq,
                        acc[r]);
        }
    }
}

// ---- pair mode (32 rows) ----
// At 32 rows the tile arithmetic reads 2 x 4 activation pieces and 2 x 2 row
// sums from LDS per lane, 12 KB per wave and tile, about what a CU's LDS
// delivers while HBM delivers the tile.  So a wave works on two of its
// rowblocks at once: a batch is 2 tiles of each, and every activation read
// feeds both rowblocks.

// One tile (index pl of the staged segment) of rowblocks a and b: the scale
// terms (the bias terms follow per pair of tiles, ss_bias2_pair).
template <int MT>
__device__ __forceinline__ void ss_tile2(u32x4_t ca, u32x2_t sba, u32x4_t cb, u32x2_t sbb,
                                         const uint16_t *xl, int pl, int lane,
                                         const Q4Consts &kq, f32x4_t acc_a[MT],
                                         f32x4_t acc_b[MT]) {
    typedef SsCfg<MT> C;
    const int kg = lane >> 4, r16 = lane & 15;
    bf16x8_t Ba[4], Bb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        Ba[q] = q4_word_to_bf16x8(ca[q], kq);
        Bb[q] = q4_word_to_bf16x8(cb[q], kq);
    }
    const float sa0 = f16_lo(sba[0]), sa1 = f16_lo(sba[1]);
    const float sb0 = f16_lo(sbb[0]), sb1 = f16_lo(sbb[1]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const uint16_t *ar = xl + (16 * mt + r16) * C::RS + pl * 128 + 8 * kg;
        bf16x8_t A[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) A[q] = *reinterpret_cast<const bf16x8_t *>(ar + 32 * q);
        const f32x4_t Z = {0.f, 0.f, 0.f, 0.f};
        f32x4_t Ca0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], Ba[0], Z, 0, 0, 0);
        f32x4_t Cb0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], Bb[0], Z, 0, 0, 0);
        f32x4_t Ca1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[2], Ba[2], Z, 0, 0, 0);
        f32x4_t Cb1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[2], Bb[2], Z, 0, 0, 0);
        Ca0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1], Ba[1], Ca0, 0, 0, 0);
        Cb0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1], Bb[1], Cb0, 0, 0, 0);
        Ca1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[3], Ba[3], Ca1, 0, 0, 0);
        Cb1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[3], Bb[3], Cb1, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc_a[mt][e] = fmaf(sa1, Ca1[e], fmaf(sa0, Ca0[e], acc_a[mt][e]));
            acc_b[mt][e] = fmaf(sb1, Cb1[e], fmaf(sb0, Cb0[e], acc_b[mt][e]));
        }
    }
}

// ss_bias2 for rowblocks a and b at once: one read of the row sums of X
// feeds both.
template <int MT>
__device__ __forceinline__ void ss_bias2_pair(const SsBatch &B, const float *xs, int pl, int lane,
                                              f32x4_t acc_a[MT], f32x4_t acc_b[MT]) {
    typedef SsCfg<MT> C;
    const int kg = lane >> 4, r16 = lane & 15;
    const bool hi = kg & 1, t1 = kg & 2;
    const unsigned wa = t1 ? (hi ? B.sb[1][1] : B.sb[1][0]) : (hi ? B.sb[0][1] : B.sb[0][0]);
    const unsigned wb = t1 ? (hi ? B.sb[3][1] : B.sb[3][0]) : (hi ? B.sb[2][1] : B.sb[2][0]);
    const float ba = fmaf(-128.f, f16_lo(wa), f16_hi(wa));
    const float bb = fmaf(-128.f, f16_lo(wb), f16_hi(wb));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const float x = xs[(2 * pl + kg) * C::MP + 16 * mt + r16];
        acc_a[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(x, ba, acc_a[mt], 0, 0, 0);
        acc_b[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(x, bb, acc_b[mt], 0, 0, 0);
    }
}

// Issue tile j's loads of the next batch (tiles nb0, nb0 + 1 of rowblocks a
// and b into N: slots j and 2 + j), then tile j's arithmetic of batch B; the
// bias terms of both tiles after the second.
template <int MT>
__device__ __forceinline__ void sp_step(SsBatch &N, __amdgpu_buffer_rsrc_t ra,
                                        __amdgpu_buffer_rsrc_t rb, int nb0, int pn,
                                        const SsBatch &B, int pl0, const uint16_t *xl,
                                        const float *xs, int lane, const Q4Consts &kq,
                                        f32x4_t acc_a[MT], f32x4_t acc_b[MT]) {
    const unsigned lc = 16u * lane, ls = 1024u + 8u * (lane & 15);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        __builtin_amdgcn_sched_barrier(0);
        const unsigned to = (unsigned)min(nb0 + j, pn - 1) * Q4_TILE_BYTES;
        N.c[j] = buf_ld_x4(ra, lc, to);
        N.sb[j] = buf_ld_x2(ra, ls, to);
        N.c[2 + j] = buf_ld_x4(rb, lc, to);
        N.sb[2 + j] = buf_ld_x2(rb, ls, to);
        // the loads stay here; ALU, MFMA and LDS work may move across, so
        // the scheduler can overlap one tile's MFMA latency with the next
        // tile's unpacking (mask: everything but vector memory)
        __builtin_amdgcn_sched_barrier(0x078F);
        ss_tile2<MT>(B.c[j], B.sb[j], B.c[2 + j], B.sb[2 + j], xl, pl0 + j, lane, kq, acc_a,
                     acc_b);
    }
    ss_bias2_pair<MT>(B, xs, pl0, lane, acc_a, acc_b);
}

// The first batch (tiles 0, 1 of the segment) of rowblocks a and b.
__device__ __forceinline__ void sp_first(SsBatch &A, const WorkItem &it, int rba, int rbb,
                                         int pbase, int pn, bool va, bool vb, int lane) {
    const __amdgpu_buffer_rsrc_t ra = ss_rsrc(it, rba, pbase, pn, va);
    const __amdgpu_buffer_rsrc_t rb = ss_rsrc(it, rbb, pbase, pn, vb);
    const unsigned lc = 16u * lane, ls = 1024u + 8u * (lane & 15);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const unsigned to = (unsigned)min(j, pn - 1) * Q4_TILE_BYTES;
        A.c[j] = buf_ld_x4(ra, lc, to);
        A.sb[j] = buf_ld_x2(ra, ls, to);
        A.c[2 + j] = buf_ld_x4(rb, lc, to);
        A.sb[2 + j] = buf_ld_x2(rb, ls, to);
    }
}

// This wave's rowblocks i0 .. i0 + n - 1 (n <= R, R even) in pairs; the
// wave's rowblock i is first + WAVES * i and exists while i < mine.  A holds
// the first batch of the pair (i0, i0 + 1) on entry; the last step of a pair
// loads the next pair's first batch: the next pair of the block, or, when
// `cross`, the first pair of the next block.  Pairs past the wave's rowblocks
// read through empty buffers (zero) and are not stored.
template <int MT, int R>
__device__ __forceinline__ void ss_block_pair(SsBatch &A, SsBatch &B, const WorkItem &it,
                                              int first, int i0, int n, int mine, bool cross,
                                              int pbase, int pn, const uint16_t *xl,
                                              const float *xs, int lane, const Q4Consts &kq,
                                              f32x4_t acc[R][MT]) {
    typedef SsCfg<MT> C;
    static_assert(R % 2 == 0, "pairs");
    const int nb = (pn + 1) / 2, nbe = nb + (nb & 1);  // batches of 2 tiles, even count
#pragma unroll
    for (int p = 0; p < R / 2; ++p) {
        if (2 * p >= n) break;  // uniform
        const int ia = i0 + 2 * p;
        const int rba = first + C::WAVES * ia, rbb = rba + C::WAVES;
        const bool vb = 2 * p + 1 < n;
        const bool inblock = 2 * p + 2 < n;
        const int ina = ia + 2;
        const bool vna = (inblock || cross) && ina < mine;
        const bool vnb = inblock ? (2 * p + 3 < n) : (cross && ina + 1 < mine);
        const int rbna = first + C::WAVES * ina, rbnb = rbna + C::WAVES;
#pragma unroll 1
        for (int b = 0; b < nbe; b += 2) {
            sp_step<MT>(B, ss_rsrc(it, rba, pbase, pn, b + 1 < nb),
                        ss_rsrc(it, rbb, pbase, pn, vb && b + 1 < nb), 2 * (b + 1), pn, A, 2 * b,
                        xl, xs, lane, kq, acc[2 * p], acc[2 * p + 1]);
            const bool more = b + 2 < nbe;
            sp_step<MT>(A,
                        more ? ss_rsrc(it, rba, pbase, pn, b + 2 < nb)
                             : ss_rsrc(it, rbna, pbase, pn, vna),
                        more ? ss_rsrc(it, rbb, pbase, pn, vb && b + 2 < nb)
                             : ss_rsrc(it, rbnb, pbase, pn, vnb),
                        more ? 2 * (b + 2) : 0, pn, B, 2 * (b + 1), xl, xs, lane, kq,
                        acc[2 * p], acc[2 * p + 1]);
        }
    }
}

template <int MT>
__device__ __forceinline__ void ss_zero_block(f32x4_t acc[SsCfg<MT>::R][MT]) {
#pragma unroll
    for (int r = 0; r < SsCfg<MT>::R; ++r) ss_zero<MT>(acc[r]);
}

// ---- staged output (16 rows, bf16) ----
// The results of a block of rowblocks are written through LDS: each wave
// puts its rowblocks' 16 x 16 bf16 results into a staging buffer, and the
// workgroup then stores the block's rowblocks, which are consecutive, as
// runs of 16 bytes that cover whole cache lines of each output row (768
// outputs = 1536 contiguous bytes per row and half block), instead of 32-byte
// pieces of 16 rows per rowblock.  The staging buffer holds half a block
// (WAVES * SS_STG_R rowblocks), so a block is stored in two halves.
constexpr int SS_STG_R = 3;                          // rowblocks per wave and half block
constexpr int SS_STG_N = 16 * SsCfg<1>::WAVES * SS_STG_R;  // outputs per row in the buffer
constexpr int SS_STG_RS = SS_STG_N + 8;              // row stride (16-byte pad)
static_assert(SsCfg<1>::R == 2 * SS_STG_R, "a block is two staged halves");
static_assert(SsCfg<1>::LDS + (size_t)16 * SS_STG_RS * 2 <= 160 * 1024, "LDS budget");

// Whether the items' outputs can go through the staging buffer: 16 rows at
// most, bf16 output, every output row 16-byte aligned.
__device__ __forceinline__ bool ss_staged(const WorkItem &it) {
    return !it.out_f32 && (it.N % 8) == 0 && (reinterpret_cast<uintptr_t>(it.y) & 15) == 0 &&
           it.N <= (1 << 26);  // 16 output rows span less than 2^31 bytes (buffer offsets)
}

// Store this block's results (rowblocks first + WAVES * (i0 + r), r < n, of
// every wave; the block's rowblocks are [rb0, rb0 + WAVES * R) clipped to
// u1) through the staging buffer.  Every wave of the workgroup calls this
// with the same rb0 (the barriers inside are workgroup-wide).
template <int R>
__device__ __forceinline__ void ss_store_staged(const WorkItem &it, int rb0, int u1, int M, int n,
                                                const f32x4_t acc[R][1], uint16_t *stg, int tid,
                                                int lane, int wave) {
    typedef SsCfg<1> C;
    const int r16 = lane & 15, kg = lane >> 4;
    const int nend = min(u1 * RB, it.N);
    // whole-line runs go out as buffer stores with the sc1 cache bit, which
    // the pass ran 0.4% faster with than the non-temporal hint (no hint:
    // 3% slower)
    const __amdgpu_buffer_rsrc_t ry =
        make_rsrc(uniform_ptr(static_cast<const uint8_t *>(it.y)), (unsigned)M * (unsigned)it.N * 2u);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        __syncthreads();  // the previous half's stores have read the buffer
#pragma unroll
        for (int r = SS_STG_R * h; r < SS_STG_R * (h + 1); ++r) {
            if (r < n) {
                const int p = wave + C::WAVES * (r - SS_STG_R * h);  // rowblock within the half
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    stg[(4 * kg + e) * SS_STG_RS + 16 * p + r16] = f32_to_bf16(acc[r][0][e]);
            }
        }
        __syncthreads();
        const int n0 = (rb0 + C::WAVES * SS_STG_R * h) * RB;  // first output of the half
        constexpr int CH = SS_STG_N / 8;                     // 16-byte chunks per row
        for (int c = tid; c < 16 * CH; c += C::THREADS) {
            const int m = c / CH, q = c - m * CH;
            const int nn = n0 + 8 * q;
            if (m >= M || nn >= nend) continue;
            const uint16_t *src = stg + m * SS_STG_RS + 8 * q;
            const size_t o = (size_t)m * it.N + nn;
            if (nn + 8 <= nend) {
                __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4_t *>(src), ry,
                                                       (int)(2 * o), 0, 16);
            } else {
                for (int j = 0; j < nend - nn; ++j) st_global<uint16_t>(it.y, o + j, src[j]);
            }
        }
    }
}

// Rowblocks [u0, u1) of one matrix; wave w owns rowblocks u0 + w + WAVES * i.
// Results are kept in registers for R rowblocks and stored together (a store
// in the middle of the load stream makes the wave wait for loads issued
// before it).
template <int MT>
__device__ __forceinline__ void ss_range(const WorkItem &it, int u0, int u1, int M, uint16_t *xl,
                                         float *xs, uint16_t *stg, int tid, int lane, int wave,
                                         const Q4Consts &kq) {
    typedef SsCfg<MT> C;
    constexpr int R = C::R;
    const uint16_t *X = reinterpret_cast<const uint16_t *>(it.x);
    const int nseg = (it.P + C::SEGK - 1) / C::SEGK;
    const int first = u0 + wave;
    SsBatch A, B;
    f32x4_t acc[R][MT];
    if (nseg == 1) {
        // the whole K is one segment: X is staged once and every wave streams
        // all of its rowblocks without a barrier
        const int pn = it.P, nbe = ss_batches_even(pn);
        const int mine = (u1 - u0 > wave) ? (u1 - u0 - wave + C::WAVES - 1) / C::WAVES : 0;
        if constexpr (C::PAIR)
            sp_first(A, it, first, first + C::WAVES, 0, pn, mine > 0, mine > 1, lane);
        else
            ss_first(A, it, first, 0, pn, mine > 0, lane);
        __syncthreads();  // nobody still reads the previous range's X
        ss_stage<MT>(X, M, it.K, 0, nbe * SS_TPB, xl, xs, tid);
        // staged: blocks of WAVES * R consecutive rowblocks, the same number
        // for every wave (the staged store is workgroup-wide); otherwise each
        // wave runs through its own rowblocks
        const bool staged = !C::PAIR && ss_staged(it);
        const int blocks = staged ? (u1 - u0 + C::WAVES * R - 1) / (C::WAVES * R)
                                  : (mine + R - 1) / R;
#pragma unroll 1
        for (int bi = 0; bi < blocks; ++bi) {
            const int i0 = bi * R;
            const int n = max(0, min(R, mine - i0));
            ss_zero_block<MT>(acc);
            if (n > 0) {
                if constexpr (C::PAIR)
                    ss_block_pair<MT, R>(A, B, it, first, i0, n, mine, true, 0, pn, xl, xs, lane,
                                         kq, acc);
                else
                    ss_block<MT, R>(A, B, it, first, i0, n, i0 + n < mine, 0, pn, xl, xs, lane,
                                    kq, acc);
            }
            if constexpr (!C::PAIR) {
                if (staged) {
                    ss_store_staged<R>(it, u0 + C::WAVES * i0, u1, M, n, acc, stg, tid, lane,
                                       wave);
                    continue;
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (r < n) ss_store<MT>(it, first + C::WAVES * (i0 + r), M, acc[r], lane);
        }
        return;
    }
    // K spans several segments: blocks of WAVES * R rowblocks whose sums stay
    // in registers across the segments; X is staged once per block and segment
#pragma unroll 1
    for (int ub = u0; ub < u1; ub += C::WAVES * R) {
        const int left = u1 - ub;
        const int n = min(R, (left > wave) ? (left - wave + C::WAVES - 1) / C::WAVES : 0);
        const int i0 = (ub - u0) / C::WAVES;
        ss_zero_block<MT>(acc);
#pragma unroll 1
        for (int seg = 0; seg < nseg; ++seg) {
            const int pbase = seg * C::SEGK;
            const int pn = min(C::SEGK, it.P - pbase), nbe = ss_batches_even(pn);
            if constexpr (C::PAIR)
                sp_first(A, it, first + C::WAVES * i0, first + C::WAVES * (i0 + 1), pbase, pn,
                         n > 0, n > 1, lane);
            else
                ss_first(A, it, first + C::WAVES * i0, pbase, pn, n > 0, lane);
            __syncthreads();  // nobody still reads the previous segment of X
            ss_stage<MT>(X, M, it.K, seg, nbe * SS_TPB, xl, xs, tid);
            if constexpr (C::PAIR)
                ss_block_pair<MT, R>(A, B, it, first, i0, n, i0 + n, false, pbase, pn, xl, xs,
                                     lane, kq, acc);
            else
                ss_block<MT, R>(A, B, it, first, i0, n, false, pbase, pn, xl, xs, lane, kq, acc);
        }
        if constexpr (!C::PAIR) {
            if (ss_staged(it)) {
                ss_store_staged<R>(it, ub, u1, M, n, acc, stg, tid, lane, wave);
                continue;
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (r < n) ss_store<MT>(it, first + C::WAVES * (i0 + r), M, acc[r], lane);
    }
}

template <bool LIST, int MT>
__global__ void __launch_bounds__(SsCfg<MT>::THREADS, 1)
q4_skinny_stream_kernel(const WorkItem *__restrict__ items, const WorkStart *__restrict__ starts,
                        WorkItem single, int M) {
    typedef SsCfg<MT> C;
    __shared__ __attribute__((aligned(16))) uint16_t xl[C::MP * C::RS];
    __shared__ __attribute__((aligned(16))) float xs[2 * C::SEGK * C::MP];
    __shared__ __attribute__((aligned(16))) uint16_t stg[MT == 1 ? 16 * SS_STG_RS : 8];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Q4Consts kq = q4_consts();
    const int wg = xcd_work_index(blockIdx.x, gridDim.x);
    if (!LIST) {
        const int64_t n = single.units, g = gridDim.x, j = wg;
        const int u0 = (int)(j * n / g), u1 = (int)((j + 1) * n / g);
        if (u0 < u1) ss_range<MT>(single, u0, u1, M, xl, xs, stg, tid, lane, wave, kq);
        return;
    }
    const WorkStart s = starts[wg], e = starts[wg + 1];
#pragma unroll 1
    for (int i = s.item; i < e.item || (i == e.item && e.unit > 0); ++i) {
        const WorkItem it = items[i];
        const int u0 = (i == s.item) ? s.unit : 0;
        const int u1 = (i == e.item) ? e.unit : it.units;
        if (u0 < u1) ss_range<MT>(it, u0, u1, M, xl, xs, stg, tid, lane, wave, kq);
    }
}

int q4_skinny_stream_wgs_per_cu() { return 1; }

// A single matrix goes to the streaming kernel when every wave of a
// one-per-CU grid gets at least two rowblocks.
bool q4_skinny_stream_fits(int64_t N, int cus) {
    return ceil_div(N, RB) >= (int64_t)2 * SsCfg<1>::WAVES * cus;
}

hipError_t launch_q4_skinny_stream(const uint8_t *packed, const uint16_t *X, void *Y, int64_t M,
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
    const int grid = (int)(it.units < cus ? it.units : cus);
    if (M <= 16)
        hipLaunchKernelGGL((q4_skinny_stream_kernel<false, 1>), dim3(grid), dim3(SsCfg<1>::THREADS),
                           0, s, (const WorkItem *)nullptr, (const WorkStart *)nullptr,
                           it, (int)M);
    else
        hipLaunchKernelGGL((q4_skinny_stream_kernel<false, 2>), dim3(grid), dim3(SsCfg<2>::THREADS),
                           0, s, (const WorkItem *)nullptr, (const WorkStart *)nullptr,
                           it, (int)M);
    return hipGetLastError();
}

hipError_t launch_q4_skinny_stream_list(const WorkItem *items, const WorkStart *starts, int grid,
                                        int64_t M, hipStream_t s) {
    WorkItem none{};
    if (M <= 16)
        hipLaunchKernelGGL((q4_skinny_stream_kernel<true, 1>), dim3(grid), dim3(SsCfg<1>::THREADS),
                           0, s, items, starts, none, (int)M);
    else
        hipLaunchKernelGGL((q4_skinny_stream_kernel<true, 2>), dim3(grid), dim3(SsCfg<2>::THREADS),
                           0, s, items, starts, none, (int)M);
    return hipGetLastError();
}

}  // namespace qg
