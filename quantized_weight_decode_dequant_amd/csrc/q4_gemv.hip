// Decode GEMV, one activation row, 4-bit asymmetric group-64 weights:
//     y[n] = sum_g ( s[n,g] * sum_{k in g} q[n,k] x[k]  +  b[n,g] * sum_{k in g} x[k] )
// which is sum_k (s*q + b) x with the weight dequantized in registers and
// never stored ("MLX Runner: An Inference Engine You Can Read", section
// "Architecture: one command buffer per token": weight = scale x code + bias;
// Uzu page, section "Why batch-one decoding is memory-bound": every weight is
// streamed once with about one multiply-add).
//
// Work split.  A workgroup owns a contiguous range of rowblocks (16 rows
// each) and walks it in blocks of up to 64 rowblocks.  A block's work is a
// sequence of batches, one batch = 4 consecutive 128-k tiles of one rowblock
// (4.5 KB; each lane reads one 16-byte slot per tile = 32 codes of one row,
// one 64-lane load covers 16 rows x 128 k = 1 KB contiguous).  Every fourth
// batch goes to the same wave, which streams its batches double-buffered:
// the load of each tile of its next batch is issued just before the
// arithmetic of the same tile of the current batch, so each wave keeps one
// to two batches in flight, and a load that the memory pipeline cannot yet
// accept stalls one tile of arithmetic, not a batch.  The first batch is
// issued before x is staged.  x is staged in LDS in segments of 12288 k
// (every projection of a decode step is one segment) together with
// per-(tile, group, k-slice) partial sums of x, which carry the bias term.
// A wave sums its batches of one rowblock in registers, folds the four
// k-slices with two xor shuffles and adds the 16 row sums into its own LDS
// slot of the rowblock; no barrier is needed until the block ends, when the
// workgroup adds the four wave slots in wave order (deterministic) and
// writes the block's rows with coalesced stores.
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

constexpr int GV_WAVES = 4;
constexpr int GV_TPW = 4;                     // tiles per batch
constexpr int GV_THREADS = GV_WAVES * 64;
constexpr int GV_SEG_TILES = 96;              // 12288 k per staged segment
constexpr int GV_RMAX = 64;                   // rowblocks per output block
constexpr int GV_WGS_PER_CU = 5;              // resident workgroups per CU (register bound)

int q4_gemv_wgs_per_cu() { return GV_WGS_PER_CU; }

constexpr size_t GV_LDS_X = (size_t)GV_SEG_TILES * 256;      // bf16 x of a segment
constexpr size_t GV_LDS_XSUM = (size_t)GV_SEG_TILES * 32;    // [tile][group][k-slice]
constexpr size_t GV_LDS_PART = (size_t)GV_RMAX * GV_WAVES * 16 * 4;

size_t q4_gemv_lds_bytes(int64_t kmax) {
    (void)kmax;  // independent of K: x is staged one segment at a time
    return GV_LDS_X + GV_LDS_XSUM + GV_LDS_PART;
}

struct GemvLds {
    unsigned *xl;   // bf16 pairs of the staged segment [96*64]
    float *xsum;    // [96*8]
    float *part;    // [GV_RMAX][GV_WAVES][16] per-wave row sums of the block
};

// Stage tiles [0, nt) of segment `seg` of x (zero past K; nt covers the
// segment's tiles rounded up to whole batches) and their per-(tile, group,
// k-slice) sums.  Ends with a barrier; the caller guarantees no wave still
// reads the previous segment.
__device__ __forceinline__ void gv_stage_x(const GemvLds &L, const uint16_t *x, int K, int seg,
                                           int nt, int tid) {
    const int k0 = seg * GV_SEG_TILES * Q4_TILE_K;
    const int n4 = nt * 16;                    // uint4 to stage
    const int nx4 = (K - k0) / 8;              // valid uint4 (K is a multiple of 64)
    constexpr int U = (GV_SEG_TILES * 16) / GV_THREADS;  // 6
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = tid + u * GV_THREADS;
        v[u] = (i < nx4 && i < n4) ? ld_global(reinterpret_cast<const u32x4_t *>(x + k0) + i)
                                   : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = tid + u * GV_THREADS;
        if (i < n4) reinterpret_cast<u32x4_t *>(L.xl)[i] = v[u];
    }
    __syncthreads();
    for (int i = tid; i < nt * 8; i += GV_THREADS) {
        const int p = i >> 3, t = (i >> 2) & 1, kg = i & 3;
        float s = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint4 w = reinterpret_cast<const uint4 *>(L.xl)[16 * p + 8 * t + 4 * h + kg];
            s += bf16_lo(w.x) + bf16_hi(w.x) + bf16_lo(w.y) + bf16_hi(w.y) + bf16_lo(w.z) +
                 bf16_hi(w.z) + bf16_lo(w.w) + bf16_hi(w.w);
        }
        L.xsum[i] = s;
    }
    __syncthreads();
}
static_assert(GV_SEG_TILES % GV_TPW == 0, "segments hold whole batches");

// One tile's contribution of this lane (16 codes per group, 2 groups).  xp
// points at the tile's staged x for this lane's k-slice, xs at its x sums.
// d starts at -128 * sum x so that the dot products of (128 + q) with x
// leave sum q x; then acc += s * d + b * sum x per group.
__device__ __forceinline__ float gv_tile(u32x4_t c, u32x2_t sb, const uint4 *xp, const float *xs,
                                         const Q4Consts &magic, float acc) {
    const uint4 xa0 = xp[0], xb0 = xp[4], xa1 = xp[8], xb1 = xp[12];
    const float xs0 = xs[0], xs1 = xs[4];
    unsigned q[4];
    float d0 = -128.f * xs0, d1 = -128.f * xs1;
    q4_unpack(c[0], magic, q);
    d0 = dot2_bf16(q[0], xa0.x, d0);
    d0 = dot2_bf16(q[1], xa0.y, d0);
    d0 = dot2_bf16(q[2], xa0.z, d0);
    d0 = dot2_bf16(q[3], xa0.w, d0);
    q4_unpack(c[1], magic, q);
    d0 = dot2_bf16(q[0], xb0.x, d0);
    d0 = dot2_bf16(q[1], xb0.y, d0);
    d0 = dot2_bf16(q[2], xb0.z, d0);
    d0 = dot2_bf16(q[3], xb0.w, d0);
    q4_unpack(c[2], magic, q);
    d1 = dot2_bf16(q[0], xa1.x, d1);
    d1 = dot2_bf16(q[1], xa1.y, d1);
    d1 = dot2_bf16(q[2], xa1.z, d1);
    d1 = dot2_bf16(q[3], xa1.w, d1);
    q4_unpack(c[3], magic, q);
    d1 = dot2_bf16(q[0], xb1.x, d1);
    d1 = dot2_bf16(q[1], xb1.y, d1);
    d1 = dot2_bf16(q[2], xb1.z, d1);
    d1 = dot2_bf16(q[3], xb1.w, d1);
    acc = fmaf(f16_lo(sb[0]), d0, acc);
    acc = fmaf(f16_hi(sb[0]), xs0, acc);
    acc = fmaf(f16_lo(sb[1]), d1, acc);
    acc = fmaf(f16_hi(sb[1]), xs1, acc);
    return acc;
}

// Position of a wave's batch within the block: rowblock r (relative to the
// block start) and batch b of that rowblock's segment.
struct GvCursor {
    int r, b;
};

__device__ __forceinline__ GvCursor gv_advance(GvCursor c, int nb) {
    c.b += GV_WAVES;
    while (c.b >= nb) {  // uniform; at most GV_WAVES steps
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
__device__ __forceinline__ void gv_step(GvBatch &N, const WorkItem &it, int ub, int pbase, int pn,
                                        GvCursor cn, bool valid, const GvBatch &B, GvCursor c,
                                        int nb, const GemvLds &L, int lane, int wave,
                                        const Q4Consts &magic, float &acc) {
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
        acc = gv_tile(B.c[j], B.sb[j], xp + 16 * j, xs + 8 * j, magic, acc);
    }
    if (c.b + GV_WAVES >= nb) {
        acc += __shfl_xor(acc, 16);
        acc += __shfl_xor(acc, 32);
        if (lane < 16) L.part[(c.r * GV_WAVES + wave) * 16 + lane] += acc;
        acc = 0.f;
    }
}

// Rowblocks [u0, u1) of one matrix, in blocks of GV_RMAX: for every segment
// of K, stage that slice of x once and stream the block's batches.
__device__ __forceinline__ void gv_range(const WorkItem &it, int u0, int u1, const GemvLds &L,
                                         int tid, int lane, int wave, const Q4Consts &magic) {
    const int nseg = (it.P + GV_SEG_TILES - 1) / GV_SEG_TILES;
    const uint16_t *x = reinterpret_cast<const uint16_t *>(it.x);
#pragma unroll 1
    for (int ub = u0; ub < u1; ub += GV_RMAX) {
        const int nr = min(u1 - ub, GV_RMAX);
        __syncthreads();  // the previous block's partial sums have been written out
        for (int i = tid; i < nr * GV_WAVES * 16; i += GV_THREADS) L.part[i] = 0.f;
#pragma unroll 1
        for (int seg = 0; seg < nseg; ++seg) {
            const int pbase = seg * GV_SEG_TILES;
            const int pn = min(GV_SEG_TILES, it.P - pbase);
            const int nb = (pn + GV_TPW - 1) / GV_TPW;
            const int T = nr * nb;  // batches of the block in this segment
            // wave w takes the batches whose absolute index (rowblock * nb +
            // batch) is w mod GV_WAVES, so how a rowblock's batches are split over
            // the waves, and hence its rounding, does not depend on where the
            // workgroup's range starts (single and grouped launches agree
            // bit for bit)
            int t = (wave - (int)(((int64_t)ub * nb) % GV_WAVES) + GV_WAVES) % GV_WAVES;
            GvCursor ca = {t / nb, t % nb};
            GvBatch A, B;
            float acc = 0.f;
            gv_load(A, it, ub, pbase, pn, ca, t < T, lane);
            __syncthreads();  // nobody still reads the previous segment
            gv_stage_x(L, x, it.K, seg, nb * GV_TPW, tid);
#pragma unroll 1
            for (;;) {
                if (t >= T) break;
                const GvCursor cb = gv_advance(ca, nb);
                gv_step(B, it, ub, pbase, pn, cb, t + GV_WAVES < T, A, ca, nb, L, lane, wave, magic, acc);
                if (t + GV_WAVES >= T) break;
                const GvCursor cc = gv_advance(cb, nb);
                gv_step(A, it, ub, pbase, pn, cc, t + 2 * GV_WAVES < T, B, cb, nb, L, lane, wave, magic, acc);
                t += 2 * GV_WAVES;
                ca = cc;
            }
        }
        // the block's finished rows, written once by the whole workgroup (no
        // global store between the loads of the sweep above)
        __syncthreads();
        const int r0 = ub * RB, nrow = min((ub + nr) * RB, it.N) - r0;
        for (int r = tid; r < nrow; r += GV_THREADS) {
            const float *pp = L.part + ((r >> 4) * GV_WAVES) * 16 + (r & 15);
            float v = pp[0];
#pragma unroll
            for (int w = 1; w < GV_WAVES; ++w) v += pp[16 * w];
            if (it.out_f32)
                st_global<float>(it.y, (size_t)r0 + r, v);
            else
                st_global<uint16_t>(it.y, (size_t)r0 + r, f32_to_bf16(v));
        }
    }
}

// at most 168 VGPRs: 3 waves per SIMD, 3 workgroups of 4 waves per CU
// LIST = false: one matrix (`single`); LIST = true: the work list.  Two
// instantiations, so profiles tell a whole decode step from single GEMVs.
template <bool LIST>
__global__ void __launch_bounds__(GV_THREADS, GV_WGS_PER_CU)
q4_gemv_kernel(const WorkItem *__restrict__ items, const WorkStart *__restrict__ starts,
               WorkItem single) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    GemvLds L;
    L.xl = reinterpret_cast<unsigned *>(smem);
    L.xsum = reinterpret_cast<float *>(smem + GV_LDS_X);
    L.part = reinterpret_cast<float *>(smem + GV_LDS_X + GV_LDS_XSUM);
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Q4Consts magic = q4_consts();
    if (!LIST) {
        // single matrix: a contiguous share of the rowblocks per workgroup
        const int64_t n = single.units, g = gridDim.x, j = blockIdx.x;
        gv_range(single, (int)(j * n / g), (int)((j + 1) * n / g), L, tid, lane, wave, magic);
        return;
    }
    const WorkStart s = starts[blockIdx.x], e = starts[blockIdx.x + 1];
#pragma unroll 1
    for (int i = s.item; i < e.item || (i == e.item && e.unit > 0); ++i) {
        const WorkItem it = items[i];
        const int u0 = (i == s.item) ? s.unit : 0;
        const int u1 = (i == e.item) ? e.unit : it.units;
        if (u0 < u1) gv_range(it, u0, u1, L, tid, lane, wave, magic);
    }
}

hipError_t launch_q4_gemv(const uint8_t *packed, const uint16_t *x, void *y, int64_t N,
                          int64_t K, bool out_f32, int cus, hipStream_t s) {
    WorkItem it{};
    it.packed = packed;
    it.x = x;
    it.y = y;
    it.N = (int32_t)N;
    it.K = (int32_t)K;
    it.P = (int32_t)ceil_div(K, Q4_TILE_K);
    it.units = (int32_t)ceil_div(N, RB);
    it.out_f32 = out_f32 ? 1 : 0;
    const int grid = (int)(it.units < (int64_t)cus * GV_WGS_PER_CU ? it.units : (int64_t)cus * GV_WGS_PER_CU);
    hipLaunchKernelGGL(q4_gemv_kernel<false>, dim3(grid), dim3(GV_THREADS), q4_gemv_lds_bytes(K), s,
                       (const WorkItem *)nullptr, (const WorkStart *)nullptr, it);
    return hipGetLastError();
}

hipError_t launch_q4_gemv_list(const WorkItem *items, const WorkStart *starts, int grid,
                               int64_t kmax, hipStream_t s) {
    WorkItem none{};
    hipLaunchKernelGGL(q4_gemv_kernel<true>, dim3(grid), dim3(GV_THREADS), q4_gemv_lds_bytes(kmax), s,
                       items, starts, none);
    return hipGetLastError();
}

}  // namespace qg
