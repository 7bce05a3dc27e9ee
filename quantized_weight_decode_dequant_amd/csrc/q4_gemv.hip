// Decode GEMV, one activation row, 4-bit asymmetric group-64 weights:
//     y[n] = sum_g ( s[n,g] * sum_{k in g} q[n,k] x[k]  +  b[n,g] * sum_{k in g} x[k] )
// which is sum_k (s*q + b) x with the weight dequantized in registers and
// never stored ("MLX Runner: An Inference Engine You Can Read", section
// "Architecture: one command buffer per token": weight = scale x code + bias;
// Uzu page, section "Why batch-one decoding is memory-bound": every weight is
// streamed once with about one multiply-add).
//
// Work split.  A workgroup owns a contiguous range of rowblocks (16 rows
// each); for one rowblock its 4 waves split the 128-k tiles, 8 tiles per
// wave.  Each lane reads one 16-byte slot per tile (4 words = 32 codes of one
// row); one 64-lane load covers 16 rows x 128 k = 1 KB contiguous.  K is
// processed in segments of 4096: the workgroup stages that slice of x in LDS
// (with per-(tile, group, k-slice) partial sums of x, which carry the bias
// term), sweeps up to 64 of its rowblocks, keeps their partial row sums in
// LDS and moves to the next segment.  LDS use is therefore ~14 KB whatever
// K is, which keeps 8 workgroups resident per CU.
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
constexpr int GV_TPW = 8;                     // tiles per wave per (rowblock, segment)
constexpr int GV_THREADS = GV_WAVES * 64;
constexpr int GV_SEG_TILES = GV_WAVES * GV_TPW;  // 32 tiles = 4096 k per segment
constexpr int GV_RMAX = 64;                   // rowblocks per block of partial sums
constexpr int GV_WGS_PER_CU = 5;              // resident workgroups per CU (register bound)

int q4_gemv_wgs_per_cu() { return GV_WGS_PER_CU; }

size_t q4_gemv_lds_bytes(int64_t kmax) {
    (void)kmax;  // independent of K: x is staged one 4096-k segment at a time
    return (size_t)GV_SEG_TILES * 256 + (size_t)GV_SEG_TILES * 32 + GV_RMAX * 16 * 4 +
           2 * GV_WAVES * 16 * 4;
}

struct GemvLds {
    unsigned *xl;   // bf16 pairs of the staged segment [32*64]
    float *xsum;    // [32*8]
    float *part;    // [GV_RMAX][16] partial row sums across segments
    float *red;     // [2][WAVES][16]
};

// Stage x[seg*4096 .. +4096) (zero past K) and its per-(tile, group,
// k-slice) sums.  Ends with a barrier; the caller guarantees no wave still
// reads the previous segment.
__device__ __forceinline__ void gv_stage_x(const GemvLds &L, const uint16_t *x, int K, int seg,
                                           int tid) {
    const int k0 = seg * GV_SEG_TILES * Q4_TILE_K;
    const int n4 = GV_SEG_TILES * 16;          // uint4 of the segment
    const int nx4 = (K - k0) / 8;              // valid uint4 (K is a multiple of 64)
    constexpr int U = (GV_SEG_TILES * 16) / GV_THREADS;  // 2
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = tid + u * GV_THREADS;
        v[u] = (i < nx4) ? ld_global(reinterpret_cast<const u32x4_t *>(x + k0) + i)
                         : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) reinterpret_cast<u32x4_t *>(L.xl)[tid + u * GV_THREADS] = v[u];
    (void)n4;
    __syncthreads();
    {
        const int i = tid;  // 256 threads = 32 tiles x 2 groups x 4 k-slices
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
static_assert(GV_SEG_TILES * 8 == GV_THREADS, "one x-sum per thread");

// One tile's contribution of this lane (16 codes per group, 2 groups); `pl`
// is the tile's index within the staged segment.
__device__ __forceinline__ float gv_tile(u32x4_t c, u32x2_t sb, const GemvLds &L, int pl, int kg,
                                         const Q4Consts &magic, float acc) {
    const uint4 *xp = reinterpret_cast<const uint4 *>(L.xl) + 16 * pl + kg;
    const uint4 xa0 = xp[0], xb0 = xp[4], xa1 = xp[8], xb1 = xp[12];
    unsigned q[4];
    float d0 = 0.f, d1 = 0.f;
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
    const float s0 = f16_lo(sb[0]), b0 = f16_hi(sb[0]);
    const float s1 = f16_lo(sb[1]), b1 = f16_hi(sb[1]);
    const float xs0 = L.xsum[pl * 8 + kg], xs1 = L.xsum[pl * 8 + 4 + kg];
    acc = fmaf(s0, d0, acc);
    acc = fmaf(fmaf(-128.f, s0, b0), xs0, acc);
    acc = fmaf(s1, d1, acc);
    acc = fmaf(fmaf(-128.f, s1, b1), xs1, acc);
    return acc;
}

// Segment `seg` of rowblock rb: this wave's tiles, the cross-lane and
// cross-wave sums, added to the rowblock's partial sums in LDS (segments in
// order, so the result is deterministic).
__device__ __forceinline__ void gv_rowblock_seg(const WorkItem &it, int rb, int seg, int nseg,
                                                int slot, const GemvLds &L, int lane, int wave,
                                                const Q4Consts &magic, int &par) {
    const int P = it.P, kg = lane >> 4;
    const int pbase = seg * GV_SEG_TILES;
    const int pn = min(GV_SEG_TILES, P - pbase);  // tiles in this segment
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(
        uniform_ptr(it.packed + ((size_t)rb * P + pbase) * Q4_TILE_BYTES), (unsigned)pn * Q4_TILE_BYTES);
    u32x4_t c[GV_TPW];
    u32x2_t sb[GV_TPW];
    const unsigned lc = 16u * lane, ls = 1024u + 8u * (lane & 15);
#pragma unroll
    for (int j = 0; j < GV_TPW; ++j) {
        const unsigned to = (unsigned)min(wave + j * GV_WAVES, pn - 1) * Q4_TILE_BYTES;  // tail: re-read
        c[j] = buf_ld_x4(rs, lc, to);
        sb[j] = buf_ld_x2(rs, ls, to);
    }
    // keep all of this wave's loads issued before any of the arithmetic: the
    // scheduler would otherwise move them next to their uses
    __builtin_amdgcn_sched_barrier(0);
    // no branch around the tiles (a branch would let the compiler sink each
    // load next to its use): tail tiles are computed from the clamped
    // re-read and discarded with a select
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < GV_TPW; ++j) {
        const int pl = wave + j * GV_WAVES;
        const float a = gv_tile(c[j], sb[j], L, min(pl, pn - 1), kg, magic, acc);
        acc = (pl < pn) ? a : acc;
    }
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    float *red = L.red + par * GV_WAVES * 16;
    if (lane < 16) red[wave * 16 + lane] = acc;
    __syncthreads();
    if (wave == 0 && lane < 16) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < GV_WAVES; ++w) v += red[w * 16 + lane];
        float *pp = L.part + slot * 16 + lane;
        *pp = (seg > 0) ? *pp + v : v;
    }
    par ^= 1;
}

// Rowblocks [u0, u1) of one matrix, in blocks of GV_RMAX: for every 4096-k
// segment, stage that slice of x once and sweep the block's rowblocks.
__device__ __forceinline__ void gv_range(const WorkItem &it, int u0, int u1, const GemvLds &L,
                                         int tid, int lane, int wave, const Q4Consts &magic, int &par) {
    const int nseg = (it.P + GV_SEG_TILES - 1) / GV_SEG_TILES;
    const uint16_t *x = reinterpret_cast<const uint16_t *>(it.x);
#pragma unroll 1
    for (int ub = u0; ub < u1; ub += GV_RMAX) {
        const int ue = min(u1, ub + GV_RMAX);
#pragma unroll 1
        for (int seg = 0; seg < nseg; ++seg) {
            __syncthreads();  // nobody still reads the previous segment or partials
            gv_stage_x(L, x, it.K, seg, tid);
#pragma unroll 1
            for (int u = ub; u < ue; ++u)
                gv_rowblock_seg(it, u, seg, nseg, u - ub, L, lane, wave, magic, par);
        }
        // the block's finished rows, written once by the whole workgroup (no
        // global store between the loads of the sweep above)
        __syncthreads();
        const int r0 = ub * RB, nr = min(ue * RB, it.N) - r0;
        for (int r = tid; r < nr; r += GV_THREADS) {
            const float v = L.part[r];
            if (it.out_f32)
                reinterpret_cast<float *>(it.y)[r0 + r] = v;
            else
                reinterpret_cast<uint16_t *>(it.y)[r0 + r] = f32_to_bf16(v);
        }
    }
}

// at most 95 VGPRs: 5 waves per SIMD, 5 workgroups of 4 waves per CU
// LIST = false: one matrix (`single`); LIST = true: the work list.  Two
// instantiations, so profiles tell a whole decode step from single GEMVs.
template <bool LIST>
__global__ void __launch_bounds__(GV_THREADS, GV_WGS_PER_CU)
q4_gemv_kernel(const WorkItem *__restrict__ items, const WorkStart *__restrict__ starts,
               WorkItem single) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    GemvLds L;
    L.xl = reinterpret_cast<unsigned *>(smem);
    L.xsum = reinterpret_cast<float *>(smem + (size_t)GV_SEG_TILES * 256);
    L.part = L.xsum + GV_SEG_TILES * 8;
    L.red = L.part + GV_RMAX * 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Q4Consts magic = q4_consts();
    int par = 0;
    if (!LIST) {
        // single matrix: a contiguous share of the rowblocks per workgroup
        const int64_t n = single.units, g = gridDim.x, j = blockIdx.x;
        gv_range(single, (int)(j * n / g), (int)((j + 1) * n / g), L, tid, lane, wave, magic, par);
        return;
    }
    const WorkStart s = starts[blockIdx.x], e = starts[blockIdx.x + 1];
#pragma unroll 1
    for (int i = s.item; i < e.item || (i == e.item && e.unit > 0); ++i) {
        const WorkItem it = items[i];
        const int u0 = (i == s.item) ? s.unit : 0;
        const int u1 = (i == e.item) ? e.unit : it.units;
        if (u0 < u1) gv_range(it, u0, u1, L, tid, lane, wave, magic, par);
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
