// Decode GEMV, one activation row, 4-bit asymmetric group-64 weights:
//     y[n] = sum_g ( s[n,g] * sum_{k in g} q[n,k] x[k]  +  b[n,g] * sum_{k in g} x[k] )
// which is sum_k (s*q + b) x with the weight dequantized in registers and
// never stored ("MLX Runner: An Inference Engine You Can Read", section
// "Architecture: one command buffer per token": weight = scale x code + bias;
// Uzu page, section "Why batch-one decoding is memory-bound": every weight is
// streamed once with about one multiply-add).
//
// Work split.  A workgroup owns one rowblock (16 rows) at a time; its waves
// split the rowblock's 128-k tiles.  Each lane reads one 16-byte slot per
// tile (4 words = 32 codes of one row); one 64-lane load covers 16 rows x
// 128 k = 1 KB contiguous.  x is staged in LDS together with per-(tile,
// group, k-slice) partial sums of x, which carry the bias term.
//
// Two launch modes share the body:
//  - single matrix (qgemv_run): rowblocks rb = blockIdx.x + i * gridDim.x;
//  - work list (one launch for many independent GEMVs, e.g. every projection
//    of a decode step): workgroup j walks the contiguous (matrix, rowblock)
//    range [starts[j], starts[j+1]), balanced by bytes on the host, and
//    re-stages x only when the matrix changes.
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
constexpr int GV_TPW = 8;  // tiles per wave per batch
constexpr int GV_THREADS = GV_WAVES * 64;

size_t q4_gemv_lds_bytes(int64_t kmax) {
    const int64_t P = ceil_div(kmax, Q4_TILE_K);
    return (size_t)P * 256 + (size_t)P * 32 + 2 * GV_WAVES * 16 * 4;
}

struct GemvLds {
    unsigned *xl;  // bf16 pairs [P*64]
    float *xsum;   // [P*8]
    float *red;    // [2][WAVES][16]
};

// Stage x (zero past K) and its per-(tile, group, k-slice) sums.  Ends with a
// barrier; the caller guarantees no wave still reads the previous x.
__device__ __forceinline__ void gv_stage_x(const GemvLds &L, const uint16_t *x, int K, int P,
                                           int tid) {
    constexpr int U = 8;
    const int n4 = P * 16, nx4 = K / 8;
    for (int b = tid; b < n4; b += GV_THREADS * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = b + u * GV_THREADS;
            v[u] = (i < nx4) ? reinterpret_cast<const uint4 *>(x)[i] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = b + u * GV_THREADS;
            if (i < n4) reinterpret_cast<uint4 *>(L.xl)[i] = v[u];
        }
    }
    __syncthreads();
    for (int i = tid; i < P * 8; i += GV_THREADS) {
        const int p = i >> 3, t = (i >> 2) & 1, kg = i & 3;
        float s = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint4 v = reinterpret_cast<const uint4 *>(L.xl)[16 * p + 8 * t + 4 * h + kg];
            s += bf16_lo(v.x) + bf16_hi(v.x) + bf16_lo(v.y) + bf16_hi(v.y) + bf16_lo(v.z) +
                 bf16_hi(v.z) + bf16_lo(v.w) + bf16_hi(v.w);
        }
        L.xsum[i] = s;
    }
    __syncthreads();
}

// One tile's contribution of this lane (16 codes per group, 2 groups).
__device__ __forceinline__ float gv_tile(u32x4_t c, u32x2_t sb, const GemvLds &L, int p, int kg,
                                         unsigned magic, float acc) {
    const uint4 *xp = reinterpret_cast<const uint4 *>(L.xl) + 16 * p + kg;
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
    const float xs0 = L.xsum[p * 8 + kg], xs1 = L.xsum[p * 8 + 4 + kg];
    acc = fmaf(s0, d0, acc);
    acc = fmaf(fmaf(-128.f, s0, b0), xs0, acc);
    acc = fmaf(s1, d1, acc);
    acc = fmaf(fmaf(-128.f, s1, b1), xs1, acc);
    return acc;
}

// Rowblock rb of the matrix: this wave's tiles, then the cross-wave sum.
__device__ __forceinline__ void gv_rowblock(const WorkItem &it, int rb, const GemvLds &L,
                                            int lane, int wave, unsigned magic, int &par) {
    const int P = it.P, kg = lane >> 4;
    const uint8_t *base = it.packed + (size_t)rb * P * Q4_TILE_BYTES;
    float acc = 0.f;
    for (int p0 = wave; p0 < P; p0 += GV_WAVES * GV_TPW) {
        u32x4_t c[GV_TPW];
        u32x2_t sb[GV_TPW];
#pragma unroll
        for (int j = 0; j < GV_TPW; ++j) {
            const int p = min(p0 + j * GV_WAVES, P - 1);  // tail: re-read the last tile
            const uint8_t *tb = base + (size_t)p * Q4_TILE_BYTES;
            c[j] = ld_nt(reinterpret_cast<const u32x4_t *>(tb) + lane);
            sb[j] = ld_nt(reinterpret_cast<const u32x2_t *>(tb + 1024) + (lane & 15));
        }
#pragma unroll
        for (int j = 0; j < GV_TPW; ++j) {
            const int p = p0 + j * GV_WAVES;
            if (p < P) acc = gv_tile(c[j], sb[j], L, p, kg, magic, acc);
        }
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
        const int row = rb * RB + lane;
        if (row < it.N) {
            if (it.out_f32)
                reinterpret_cast<float *>(it.y)[row] = v;
            else
                reinterpret_cast<uint16_t *>(it.y)[row] = f32_to_bf16(v);
        }
    }
    par ^= 1;
}

__global__ void __launch_bounds__(GV_THREADS)
q4_gemv_kernel(const WorkItem *__restrict__ items, const WorkStart *__restrict__ starts,
               WorkItem single, int pmax) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    GemvLds L;
    L.xl = reinterpret_cast<unsigned *>(smem);
    L.xsum = reinterpret_cast<float *>(smem + (size_t)pmax * 256);
    L.red = L.xsum + pmax * 8;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const unsigned magic = bf16_magic128x2();
    int par = 0;
    if (items == nullptr) {
        gv_stage_x(L, reinterpret_cast<const uint16_t *>(single.x), single.K, single.P, tid);
        for (int rb = blockIdx.x; rb < single.units; rb += gridDim.x)
            gv_rowblock(single, rb, L, lane, wave, magic, par);
        return;
    }
    const WorkStart s = starts[blockIdx.x], e = starts[blockIdx.x + 1];
    int i = s.item, u = s.unit, staged = -1;
    WorkItem it;
    while (i < e.item || (i == e.item && u < e.unit)) {
        if (i != staged) {
            it = items[i];
            gv_stage_x(L, reinterpret_cast<const uint16_t *>(it.x), it.K, it.P, tid);
            staged = i;
        }
        gv_rowblock(it, u, L, lane, wave, magic, par);
        if (++u == it.units) {
            ++i;
            u = 0;
        }
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
    const int grid = (int)(it.units < (int64_t)cus * 8 ? it.units : (int64_t)cus * 8);
    hipLaunchKernelGGL(q4_gemv_kernel, dim3(grid), dim3(GV_THREADS), q4_gemv_lds_bytes(K), s,
                       (const WorkItem *)nullptr, (const WorkStart *)nullptr, it, it.P);
    return hipGetLastError();
}

hipError_t launch_q4_gemv_list(const WorkItem *items, const WorkStart *starts, int grid,
                               int64_t kmax, hipStream_t s) {
    WorkItem none{};
    const int pmax = (int)ceil_div(kmax, Q4_TILE_K);
    hipLaunchKernelGGL(q4_gemv_kernel, dim3(grid), dim3(GV_THREADS), q4_gemv_lds_bytes(kmax), s,
                       items, starts, none, pmax);
    return hipGetLastError();
}

}  // namespace qg
