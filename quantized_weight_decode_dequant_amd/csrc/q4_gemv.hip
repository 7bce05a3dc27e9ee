// Decode GEMV, 4-bit asymmetric group-64 weights, on the VALU:
//     y[n] = sum_g ( s[n,g] * sum_{k in g} q[n,k] x[k]  +  b[n,g] * sum_{k in g} x[k] )
// which is sum_k (s*q + b) x with the weight dequantized in registers and
// never stored ("MLX Runner: An Inference Engine You Can Read", section
// "Architecture: one command buffer per token": weight = scale x code + bias;
// Uzu page, section "Why batch-one decoding is memory-bound": every weight is
// streamed once with about one multiply-add).
//
// Work split.  A workgroup owns a contiguous range of rowblocks (16 rows
// each) and walks it in blocks of up to 16 rowblocks.  A block's work is a
// sequence of batches, one batch = 4 consecutive 128-k tiles of one rowblock
// (4.5 KB; each lane reads one 16-byte slot per tile = 32 codes of one row,
// one 64-lane load covers 16 rows x 128 k = 1 KB contiguous).  Every fourth
// batch goes to the same wave, which streams its batches double-buffered:
// the load of each tile of its next batch is issued just before the
// arithmetic of the same tile of the current batch, so each wave keeps one
// to two batches in flight, and a load that the memory pipeline cannot yet
// accept stalls one tile of arithmetic, not a batch.  The first batch is
// issued before x is staged.  x is staged in LDS in segments of 6144 k
// together with per-(tile, group, k-slice) partial sums of x, which carry
// the bias term; with 16-rowblock blocks that keeps a workgroup at 21.5 KB
// of LDS, so LDS does not limit how many workgroups a CU holds.
// A wave sums its batches of one rowblock in registers, folds the four
// k-slices with two xor shuffles and adds the 16 row sums into its own LDS
// slot of the rowblock; no barrier is needed until the block ends, when the
// workgroup adds the four wave slots in wave order (deterministic) and
// writes the block's rows with coalesced stores.
//
// The same kernel serves a few activation rows at once (M = 2..4, staged
// side by side; 3 runs as 4 with a zero row): the codes of a tile are
// unpacked once and feed one v_dot2 chain per row, so each weight is still
// read once per call.  Past 4 rows the VALU work per byte outgrows the
// bf16 MFMA kernels, whose cost does not depend on M up to 16.
//
// Two launch modes share the body:
//  - single matrix (qgemv_run): workgroup j takes rowblocks
//    [j*n/G, (j+1)*n/G);
//  - work list (one launch for many independent GEMVs, e.g. every projection
//    of a decode step): workgroup j walks the contiguous (matrix, rowblock)
//    range [starts[j], starts[j+1]), balanced by bytes on the host.
//
// Arithmetic per word: (w >> 4j) & 0x000F000F | 0x43004300 (one
// v_and_or_b32) turns two codes into the bf16 pair (128 + q, 128 + q'),
// exact; v_dot2_f32_bf16 multiplies it with the matching x pair and adds in
// fp32.  The 128 offset is removed with the x partial sum:
// s * sum (128 + q) x + (b - 128 s) * sum x.  Lanes of one row (k-slices
// 0..3) are summed with two xor shuffles, the waves through LDS, in a fixed
// order (deterministic).
#include "qg_internal.h"

namespace qg {

constexpr int GV_TPW = 4;                     // tiles per batch
constexpr int GV_RMAX = 16;                   // rowblocks per output block
constexpr int GV_MR_MAX = 4;                  // most activation rows per launch
// Waves per workgroup: 4 for large single matrices and for 2 or 4 activation
// rows; 8 for single matrices with few rowblocks, whose workgroups each get
// one or two rowblocks (with 8 waves every batch of a 4096-k rowblock has a
// wave of its own, so a call waits on one memory latency per wave instead of
// two), and for the work list at one row: two 8-wave workgroups per CU
// stream a decode step about 1.5% faster than five 4-wave ones (each
// workgroup step reads 8 consecutive batches of its rowblock instead of 4,
// as a plain read with 8-wave workgroups outruns one with 4-wave ones).
constexpr int GV_WAVES = 4;
constexpr int GV_WAVES_SMALL = 8;

int q4_gemv_rows_max() { return GV_MR_MAX; }

// Per row count MR (1, 2 or 4 staged activation rows) and wave count W:
// tiles per staged segment (6144 k for one row; fewer for more rows, so that
// the staged x of all rows stays at 12 KB) and the LDS of one workgroup.
template <int MR, int W = GV_WAVES>
struct GvCfg {
    static constexpr int WAVES = W;
    static constexpr int THREADS = W * 64;
    static constexpr int SEG = 48 / MR;
    static constexpr int ROW4 = SEG * 16;     // uint4 of staged x per row
    static constexpr int ROWS = SEG * 8;      // x sums per row
    static constexpr size_t LDS_X = (size_t)ROW4 * 16 * MR;
    static constexpr size_t LDS_XSUM = (size_t)ROWS * 4 * MR;
    // partial-sum slots per rowblock: a batch's sums go to slot (absolute
    // batch index) mod SLOTS; one row: 8 slots for 4 or 8 waves alike, so the
    // rounding does not depend on the wave count (slot mod W is the wave)
    static constexpr int SLOTS = MR == 1 ? 8 : W;
    static_assert(SLOTS % W == 0, "a slot belongs to one wave");
    static constexpr size_t LDS_PART = (size_t)GV_RMAX * SLOTS * MR * 16 * 4;
    static constexpr size_t LDS = LDS_X + LDS_XSUM + LDS_PART;
    // resident workgroups per CU, set by registers: at most 102 VGPRs for 5
    // 4-wave workgroups (1 or 2 rows), 128 for 4 (4 rows); 8-wave
    // workgroups: 2 (at most 128 VGPRs); LDS allows more
    static constexpr int WPC = W == 4 ? (MR <= 2 ? 5 : 4) : 2;
    static_assert(SEG % GV_TPW == 0, "segments hold whole batches");
    static_assert(LDS * WPC <= 160 * 1024, "LDS must not limit residency");
};

static int gv_rows(int64_t M) { return M <= 1 ? 1 : (M <= 2 ? 2 : 4); }

int q4_gemv_wgs_per_cu(int64_t M) { return gv_rows(M) <= 2 ? GvCfg<1>::WPC : GvCfg<4>::WPC; }

int q4_gemv_list_wgs_per_cu(int64_t M) {
    return gv_rows(M) == 1 ? GvCfg<1, GV_WAVES_SMALL>::WPC : q4_gemv_wgs_per_cu(M);
}

size_t q4_gemv_lds_bytes(int64_t M) {
    const int mr = gv_rows(M);
    return mr == 1 ? GvCfg<1>::LDS : (mr == 2 ? GvCfg<2>::LDS : GvCfg<4>::LDS);
}

struct GemvLds {
    unsigned *xl;   // bf16 pairs of the staged segment, [MR][SEG*64]
    float *xsum;    // [MR][SEG*8]: per (tile, group, k-slice)
    float *part;    // [GV_RMAX][slots][MR][16] row sums of the block per batch slot
};

// Staging of tiles [0, nt) of segment `seg` of the M activation rows (rows
// past M and k past K read as zero; nt covers the segment's tiles rounded up
// to whole batches) with their per-(tile, group, k-slice) sums, in two
// halves: gv_stage_load brings the x chunks into registers, gv_stage_store
// writes them to LDS (the caller guarantees no wave still reads the previous
// segment), sums them and ends with a barrier.  The x loads go out before
// the segment's first weight loads: a wave's loads complete in issue order,
// so x issued after the weights would wait for them.
template <int MR, int W>
struct GvStage {
    static constexpr int U = (GvCfg<MR, W>::ROW4 * MR + GvCfg<MR, W>::THREADS - 1) /
                             GvCfg<MR, W>::THREADS;
    u32x4_t v[U];
};

template <int MR, int W>
__device__ __forceinline__ void gv_stage_load(GvStage<MR, W> &st, const uint16_t *x, int M, int K,
                                              int seg, int nt, int tid) {
    typedef GvCfg<MR, W> C;
    const int k0 = seg * C::SEG * Q4_TILE_K;
    const int n4 = nt * 16;                    // uint4 to stage per row
    const int nx4 = (K - k0) / 8;              // valid uint4 per row (K is a multiple of 64)
#pragma unroll
    for (int u = 0; u < GvStage<MR, W>::U; ++u) {
        const int i = tid + u * C::THREADS, m = i / C::ROW4, j = i - m * C::ROW4;
        st.v[u] = (m < M && m < MR && j < nx4 && j < n4)
                      ? ld_global(reinterpret_cast<const u32x4_t *>(x + (size_t)m * K + k0) + j)
                      : u32x4_t{0u, 0u, 0u, 0u};
    }
}

template <int MR, int W>
__device__ __forceinline__ void gv_stage_store(const GvStage<MR, W> &st, const GemvLds &L, int nt,
                                               int tid) {
    typedef GvCfg<MR, W> C;
    const int n4 = nt * 16;
#pragma unroll
    for (int u = 0; u < GvStage<MR, W>::U; ++u) {
        const int i = tid + u * C::THREADS, m = i / C::ROW4, j = i - m * C::ROW4;
        if (m < MR && j < n4) reinterpret_cast<u32x4_t *>(L.xl)[i] = st.v[u];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const uint4 *xr = reinterpret_cast<const uint4 *>(L.xl) + m * C::ROW4;
        for (int i = tid; i < nt * 8; i += C::THREADS) {
            const int p = i >> 3, t = (i >> 2) & 1, kg = i & 3;
            float s = 0.f;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint4 w = xr[16 * p + 8 * t + 4 * h + kg];
                s += bf16_lo(w.x) + bf16_hi(w.x) + bf16_lo(w.y) + bf16_hi(w.y) + bf16_lo(w.z) +
                     bf16_hi(w.z) + bf16_lo(w.w) + bf16_hi(w.w);
            }
            L.xsum[m * C::ROWS + i] = s;
        }
    }
    __syncthreads();
}

// One tile's contribution of this lane (16 codes per group, 2 groups) to
// each of the MR rows.  The codes are unpacked once and serve every row.
// xp points at the tile's staged x of row 0 for this lane's k-slice, xs at
// its x sums.  d starts at -128 * sum x so that the dot products of
// (128 + q) with x leave sum q x; then acc += s * d + b * sum x per group.
template <int MR>
__device__ __forceinline__ void gv_tile(u32x4_t c, u32x2_t sb, const uint4 *xp, const float *xs,
                                        const Q4Consts &magic, float (&acc)[MR]) {
    typedef GvCfg<MR> C;
    float d[MR][2];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        d[m][0] = -128.f * xs[m * C::ROWS];
        d[m][1] = -128.f * xs[m * C::ROWS + 4];
    }
    // word w holds 8 codes of group w >> 1; its x is uint4 4 * w of the tile
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        unsigned q[4];
        q4_unpack(c[w], magic, q);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const uint4 xv = xp[m * C::ROW4 + 4 * w];
            float &dd = d[m][w >> 1];
            dd = dot2_bf16(q[0], xv.x, dd);
            dd = dot2_bf16(q[1], xv.y, dd);
            dd = dot2_bf16(q[2], xv.z, dd);
            dd = dot2_bf16(q[3], xv.w, dd);
        }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        acc[m] = fmaf(f16_lo(sb[0]), d[m][0], acc[m]);
        acc[m] = fmaf(f16_hi(sb[0]), xs[m * C::ROWS], acc[m]);
        acc[m] = fmaf(f16_lo(sb[1]), d[m][1], acc[m]);
        acc[m] = fmaf(f16_hi(sb[1]), xs[m * C::ROWS + 4], acc[m]);
    }
}

// Position of a wave's batch within the block: rowblock r (relative to the
// block start) and batch b of that rowblock's segment.
struct GvCursor {
    int r, b;
};

template <int W>
__device__ __forceinline__ GvCursor gv_advance(GvCursor c, int nb) {
    c.b += W;
    while (c.b >= nb) {  // uniform; at most W steps
        c.b -= nb;
        ++c.r;
    }
    return c;
}

struct GvBatch {
    u32x4_t c[GV_TPW];
    u32x2_t sb[GV_TPW];
};

// Issue the loads of one batch.  A batch past the end of the wave's work
// reads through an empty buffer resource: zeros, no memory traffic.
__device__ __forceinline__ void gv_load(GvBatch &B, const WorkItem &it, int ub, int pbase, int pn,
                                        GvCursor c, bool valid, int lane) {
    const uint8_t *base = it.packed + ((size_t)(ub + c.r) * it.P + pbase) * Q4_TILE_BYTES;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(uniform_ptr(base), valid ? (unsigned)pn * Q4_TILE_BYTES : 0u);
    const unsigned lc = 16u * lane, ls = 1024u + 8u * (lane & 15);
#pragma unroll
    for (int j = 0; j < GV_TPW; ++j) {
        // tiles past the segment's end re-read its last tile (they add zero)
        const unsigned to = (unsigned)min(c.b * GV_TPW + j, pn - 1) * Q4_TILE_BYTES;
        B.c[j] = buf_ld_x4(rs, lc, to);
        B.sb[j] = buf_ld_x2(rs, ls, to);
    }
}

// One step of a wave's stream: issue the loads of its next batch N tile by
// tile, each followed by the arithmetic of the same tile of the current batch
// B, so that a load the memory pipeline cannot yet accept holds up one tile
// of arithmetic rather than a whole batch.  At the wave's last batch of a
// rowblock the row sums go to the wave's LDS slot of that rowblock.  Tiles
// past the segment's end re-read its last tile; their staged x and x sums
// are zero, so they add exactly zero.
template <int MR, int W>
__device__ __forceinline__ void gv_step(GvBatch &N, const WorkItem &it, int ub, int pbase, int pn,
                                        GvCursor cn, bool valid, const GvBatch &B, GvCursor c,
                                        int nb, int slot, const GemvLds &L, int lane,
                                        const Q4Consts &magic, float (&acc)[MR]) {
    constexpr int S = GvCfg<MR, W>::SLOTS;
    const uint8_t *base = it.packed + ((size_t)(ub + cn.r) * it.P + pbase) * Q4_TILE_BYTES;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(uniform_ptr(base), valid ? (unsigned)pn * Q4_TILE_BYTES : 0u);
    const unsigned lc = 16u * lane, ls = 1024u + 8u * (lane & 15);
    const int kg = lane >> 4;
    const uint4 *xp = reinterpret_cast<const uint4 *>(L.xl) + 16 * GV_TPW * c.b + kg;
    const float *xs = L.xsum + 8 * GV_TPW * c.b + kg;
#pragma unroll
    for (int j = 0; j < GV_TPW; ++j) {
        __builtin_amdgcn_sched_barrier(0);
        const unsigned to = (unsigned)min(cn.b * GV_TPW + j, pn - 1) * Q4_TILE_BYTES;
        N.c[j] = buf_ld_x4(rs, lc, to);
        N.sb[j] = buf_ld_x2(rs, ls, to);
        __builtin_amdgcn_sched_barrier(0);
        gv_tile<MR>(B.c[j], B.sb[j], xp + 16 * j, xs + 8 * j, magic, acc);
    }
    // the row sums into the batch's slot of the rowblock: with one row after
    // every batch (a slot holds every 8th batch, and 4 or 8 waves must add
    // the batches of a slot alike); with more rows every batch of the
    // wave's rowblock goes to the slot of the wave, which takes them after
    // its last batch of the rowblock
    if (MR == 1 || c.b + W >= nb) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            float a = acc[m];
            a += __shfl_xor(a, 16);
            a += __shfl_xor(a, 32);
            if (lane < 16) L.part[((c.r * S + slot) * MR + m) * 16 + lane] += a;
            acc[m] = 0.f;
        }
    }
}

// Rowblocks [u0, u1) of one matrix, in blocks of GV_RMAX: for every segment
// of K, stage that slice of the M activation rows once and stream the
// block's batches.
template <int MR, int W>
__device__ __forceinline__ void gv_range(const WorkItem &it, int u0, int u1, int M,
                                         const GemvLds &L, int tid, int lane, int wave,
                                         const Q4Consts &magic) {
    typedef GvCfg<MR, W> C;
    constexpr int S = C::SLOTS;
    const int nseg = (it.P + C::SEG - 1) / C::SEG;
    const uint16_t *x = reinterpret_cast<const uint16_t *>(it.x);
#pragma unroll 1
    for (int ub = u0; ub < u1; ub += GV_RMAX) {
        const int nr = min(u1 - ub, GV_RMAX);
        __syncthreads();  // the previous block's partial sums have been written out
        for (int i = tid; i < nr * S * MR * 16; i += C::THREADS) L.part[i] = 0.f;
#pragma unroll 1
        for (int seg = 0; seg < nseg; ++seg) {
            const int pbase = seg * C::SEG;
            const int pn = min(C::SEG, it.P - pbase);
            const int nb = (pn + GV_TPW - 1) / GV_TPW;
            const int T = nr * nb;  // batches of the block in this segment
            // batch t of the block has the absolute index A = ub * nb + t
            // (rowblock * nb + batch); its sums go to slot A mod S and wave
            // A mod W computes it, so neither where the workgroup's range
            // starts nor the wave count changes how a rowblock's sums are
            // rounded (single and grouped launches agree bit for bit)
            const int a0 = (int)(((int64_t)ub * nb) % S);
            int t = (wave - a0 % W + W) % W;
            GvCursor ca = {t / nb, t % nb};
            GvBatch A, B;
            float acc[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m) acc[m] = 0.f;
            GvStage<MR, W> st;
            gv_stage_load<MR, W>(st, x, M, it.K, seg, nb * GV_TPW, tid);
            gv_load(A, it, ub, pbase, pn, ca, t < T, lane);
            __syncthreads();  // nobody still reads the previous segment
            gv_stage_store<MR, W>(st, L, nb * GV_TPW, tid);
#pragma unroll 1
            for (;;) {
                if (t >= T) break;
                const GvCursor cb = gv_advance<W>(ca, nb);
                gv_step<MR, W>(B, it, ub, pbase, pn, cb, t + W < T, A, ca, nb, (a0 + t) % S, L,
                               lane, magic, acc);
                if (t + W >= T) break;
                const GvCursor cc = gv_advance<W>(cb, nb);
                gv_step<MR, W>(A, it, ub, pbase, pn, cc, t + 2 * W < T, B, cb, nb,
                               (a0 + t + W) % S, L, lane, magic, acc);
                t += 2 * W;
                ca = cc;
            }
        }
        // the block's finished rows, written once by the whole workgroup (no
        // global store between the loads of the sweep above)
        __syncthreads();
        const int r0 = ub * RB, nrow = min((ub + nr) * RB, it.N) - r0;
        for (int i = tid; i < M * nrow; i += C::THREADS) {
            const int m = i / nrow, r = i - m * nrow;
            const float *pp = L.part + (((r >> 4) * S) * MR + m) * 16 + (r & 15);
            float v = pp[0];
#pragma unroll
            for (int w = 1; w < S; ++w) v += pp[16 * MR * w];
            const size_t o = (size_t)m * it.N + r0 + r;
            if (it.out_f32)
                st_global<float>(it.y, o, v);
            else
                st_global<uint16_t>(it.y, o, f32_to_bf16(v));
        }
    }
}

// LIST = false: one matrix (`single`); LIST = true: the work list.  Separate
// instantiations, so profiles tell a whole decode step from single GEMVs.
template <bool LIST, int MR, int NW>
__global__ void __launch_bounds__(NW * 64, (GvCfg<MR, NW>::WPC))
q4_gemv_kernel(const WorkItem *__restrict__ items, const WorkStart *__restrict__ starts,
               WorkItem single, int M) {
    typedef GvCfg<MR, NW> C;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    GemvLds L;
    L.xl = reinterpret_cast<unsigned *>(smem);
    L.xsum = reinterpret_cast<float *>(smem + C::LDS_X);
    L.part = reinterpret_cast<float *>(smem + C::LDS_X + C::LDS_XSUM);
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Q4Consts magic = q4_consts();
    if (!LIST) {
        // single matrix: a contiguous share of the rowblocks per workgroup
        const int64_t n = single.units, g = gridDim.x, j = blockIdx.x;
        gv_range<MR, NW>(single, (int)(j * n / g), (int)((j + 1) * n / g), M, L, tid, lane, wave,
                         magic);
        return;
    }
    const WorkStart s = starts[blockIdx.x], e = starts[blockIdx.x + 1];
#pragma unroll 1
    for (int i = s.item; i < e.item || (i == e.item && e.unit > 0); ++i) {
        const WorkItem it = items[i];
        const int u0 = (i == s.item) ? s.unit : 0;
        const int u1 = (i == e.item) ? e.unit : it.units;
        if (u0 < u1) gv_range<MR, NW>(it, u0, u1, M, L, tid, lane, wave, magic);
    }
}

template <bool LIST>
static hipError_t gv_launch(const WorkItem *items, const WorkStart *starts, const WorkItem &it,
                            int grid, int64_t M, bool small, hipStream_t s) {
    const int mr = gv_rows(M);
    const size_t lds = q4_gemv_lds_bytes(M);
    constexpr size_t lds_small = GvCfg<1, GV_WAVES_SMALL>::LDS;
    if (mr == 1 && (small || LIST))
        hipLaunchKernelGGL((q4_gemv_kernel<LIST, 1, GV_WAVES_SMALL>), dim3(grid),
                           dim3(GV_WAVES_SMALL * 64), lds_small, s, items, starts, it, (int)M);
    else if (mr == 1)
        hipLaunchKernelGGL((q4_gemv_kernel<LIST, 1, GV_WAVES>), dim3(grid), dim3(GV_WAVES * 64),
                           lds, s, items, starts, it, (int)M);
    else if (mr == 2)
        hipLaunchKernelGGL((q4_gemv_kernel<LIST, 2, GV_WAVES>), dim3(grid), dim3(GV_WAVES * 64),
                           lds, s, items, starts, it, (int)M);
    else
        hipLaunchKernelGGL((q4_gemv_kernel<LIST, 4, GV_WAVES>), dim3(grid), dim3(GV_WAVES * 64),
                           lds, s, items, starts, it, (int)M);
    return hipGetLastError();
}

hipError_t launch_q4_gemv(const uint8_t *packed, const uint16_t *x, void *y, int64_t M, int64_t N,
                          int64_t K, bool out_f32, int cus, hipStream_t s) {
    if (M < 1 || M > GV_MR_MAX) return hipErrorInvalidValue;
    WorkItem it{};
    it.packed = packed;
    it.x = x;
    it.y = y;
    it.N = (int32_t)N;
    it.K = (int32_t)K;
    it.P = (int32_t)ceil_div(K, Q4_TILE_K);
    it.units = (int32_t)ceil_div(N, RB);
    it.out_f32 = out_f32 ? 1 : 0;
    // one activation row and at most two rowblocks per CU: 8-wave workgroups
    // of one rowblock each (see GV_WAVES_SMALL)
    const bool small = M == 1 && it.units <= (int64_t)2 * cus;
    const int64_t cap = small ? it.units : (int64_t)cus * q4_gemv_wgs_per_cu(M);
    const int grid = (int)(it.units < cap ? it.units : cap);
    return gv_launch<false>(nullptr, nullptr, it, grid, M, small, s);
}

hipError_t launch_q4_gemv_list(const WorkItem *items, const WorkStart *starts, int grid,
                               int64_t M, hipStream_t s) {
    if (M < 1 || M > GV_MR_MAX) return hipErrorInvalidValue;
    WorkItem none{};
    return gv_launch<true>(items, starts, none, grid, M, false, s);
}

}  // namespace qg
