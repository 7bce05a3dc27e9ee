// Weight-only int8 decode GEMV with one fp32 scale per row (Deltafin / Kimi K3
// page, aihot.virxact.com: the int8 resident spine, dequantized by an int8 to
// fp32 conversion fused with a row-broadcast multiply, and the packed int8
// output head that multiplies the row-int8 checkpoint directly):
//     y[n] = scale[n] * sum_k q[n][k] x[k],   q int8, x bf16, fp32 sums.
//
// Per 16-byte slot a lane flips the sign bit of every byte (u = q + 128, an
// unsigned byte), converts each byte with v_cvt_f32_ubyte{0..3} (exact) and
// accumulates u * x in fp32 against x staged in LDS as fp32; the row result is
// scale * (sum u x - 128 * sum_k x), with sum_k x taken once per workgroup in
// a fixed order.  That is 2.25 VALU operations per weight against 1 byte of
// HBM traffic.
//
// Work split as in the MXFP4 MoE streaming kernels: each workgroup takes a
// contiguous range of rowblocks; a rowblock's tiles are cut into batches of 4,
// every fourth batch of the range goes to the same wave, and each wave streams
// its batches double-buffered, the load of each tile of its next batch issued
// just before the arithmetic of the same tile of the current one.  A wave
// folds its sums of a rowblock into its own LDS slot; the workgroup adds the
// four slots in wave order when a block of up to 32 rowblocks ends
// (deterministic, no atomics).
#include "qg_internal.h"

namespace qg {

constexpr int RG_WAVES = 4;
constexpr int RG_THREADS = RG_WAVES * 64;
constexpr int RG_TPB = 4;    // tiles per batch
constexpr int RG_RMAX = 32;  // rowblocks per output block

struct RgBatch {
    u32x4_t c0[RG_TPB], c1[RG_TPB];
};

__device__ __forceinline__ void rg_tile_load(RgBatch &B, int j, __amdgpu_buffer_rsrc_t rs, int tp,
                                             int pn, int lane) {
    const unsigned to = (unsigned)min(tp, pn - 1) * Q8R_TILE_BYTES;
    B.c0[j] = buf_ld_x4(rs, 16u * lane, to);
    B.c1[j] = buf_ld_x4(rs, 1024u + 16u * lane, to);
}

// sum over the 16 bytes of c (consecutive k) of (q + 128) * x, x fp32 at xp.
__device__ __forceinline__ float rg_slot(u32x4_t c, const float4 *xp, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned u = c[i] ^ 0x80808080u;
        const float4 xv = xp[i];
        acc = fmaf((float)(u & 0xFFu), xv.x, acc);
        acc = fmaf((float)((u >> 8) & 0xFFu), xv.y, acc);
        acc = fmaf((float)((u >> 16) & 0xFFu), xv.z, acc);
        acc = fmaf((float)(u >> 24), xv.w, acc);
    }
    return acc;
}

__device__ __forceinline__ float rg_reduce_kslices(float a) {
    a += __shfl_xor(a, 16);
    a += __shfl_xor(a, 32);
    return a;
}

// LDS of one workgroup for inputs of up to kmax.
static size_t rg_lds_bytes(int64_t kmax) {
    const int64_t nb = ceil_div(ceil_div(kmax, Q8R_TILE_K), RG_TPB);
    return (size_t)nb * RG_TPB * Q8R_TILE_K * 4 + (size_t)RG_RMAX * RG_WAVES * 16 * 4 +
           (size_t)RG_THREADS * 4;
}

// Rowblocks [u0, u1) of one matrix.
__device__ __forceinline__ void rg_range(const WorkItem &it, int u0, int u1, unsigned char *smem,
                                         int tid, int lane, int wave) {
    const uint8_t *__restrict__ packed = it.packed;
    const uint16_t *__restrict__ x = reinterpret_cast<const uint16_t *>(it.x);
    const int N = it.N, K = it.K, P = it.P;
    const int kg = lane >> 4;
    const int nb = (P + RG_TPB - 1) / RG_TPB;
    const int KS = nb * RG_TPB * Q8R_TILE_K;  // staged x length (zero past K)
    float *xl = reinterpret_cast<float *>(smem);                  // [KS]
    float *part = xl + KS;                                         // [RMAX][WAVES][16]
    float *red = part + RG_RMAX * RG_WAVES * 16;                   // [THREADS]
    const size_t rb_bytes = (size_t)P * Q8R_TILE_BYTES + Q8R_RB_TAIL;
    // stage x as fp32 and take sum_k x: each thread adds its elements in k
    // order, then the threads' sums are added pairwise in a fixed tree
    __syncthreads();  // nobody still reads the previous range's x
    float own = 0.f;
    for (int k = tid; k < KS; k += RG_THREADS) {
        float v = 0.f;
        if (k < K) v = bf16_lo((unsigned)ld_global(x + k));
        xl[k] = v;
        own += v;
    }
    red[tid] = own;
    __syncthreads();
#pragma unroll
    for (int h = RG_THREADS / 2; h > 0; h >>= 1) {
        if (tid < h) red[tid] += red[tid + h];
        __syncthreads();
    }
    const float xsum = red[0];
#pragma unroll 1
    for (int ub = u0; ub < u1; ub += RG_RMAX) {
        const int nr = min(u1 - ub, RG_RMAX);
        const int T = nr * nb;
        // wave w takes the batches whose absolute index (rowblock * nb +
        // batch) is w mod RG_WAVES, so a rowblock's split over the waves,
        // and hence its rounding, does not depend on where the range starts
        // (single and grouped launches agree bit for bit)
        int t = (wave - (int)(((int64_t)ub * nb) % RG_WAVES) + RG_WAVES) % RG_WAVES;
        int ci = t / nb, cb = t % nb;
        RgBatch A, B;
        float acc = 0.f;
        {
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(
                uniform_ptr(packed + (size_t)(ub + ci) * rb_bytes),
                t < T ? (unsigned)P * Q8R_TILE_BYTES : 0u);
#pragma unroll
            for (int q = 0; q < RG_TPB; ++q) rg_tile_load(A, q, rs, cb * RG_TPB + q, P, lane);
        }
        __syncthreads();  // the previous block's partial sums are read
        for (int i = tid; i < nr * RG_WAVES * 16; i += RG_THREADS) part[i] = 0.f;
        __syncthreads();
#pragma unroll 1
        for (;;) {
            if (t >= T) break;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                RgBatch &Cur = half ? B : A;
                RgBatch &Nxt = half ? A : B;
                int ni = ci, nbx = cb + RG_WAVES;
                while (nbx >= nb) {  // uniform
                    nbx -= nb;
                    ++ni;
                }
                const bool nvalid = t + RG_WAVES < T;
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(
                    uniform_ptr(packed + (size_t)(ub + (nvalid ? ni : ci)) * rb_bytes),
                    nvalid ? (unsigned)P * Q8R_TILE_BYTES : 0u);
#pragma unroll
                for (int q = 0; q < RG_TPB; ++q) {
                    __builtin_amdgcn_sched_barrier(0);
                    rg_tile_load(Nxt, q, rs, nbx * RG_TPB + q, P, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    const float4 *xp =
                        reinterpret_cast<const float4 *>(xl + (cb * RG_TPB + q) * Q8R_TILE_K) + 4 * kg;
                    acc = rg_slot(Cur.c0[q], xp, acc);
                    acc = rg_slot(Cur.c1[q], xp + 16, acc);
                }
                if (!nvalid || ni != ci) {  // the wave's last batch of this rowblock
                    acc = rg_reduce_kslices(acc);
                    if (lane < 16) part[(ci * RG_WAVES + wave) * 16 + lane] += acc;
                    acc = 0.f;
                }
                t += RG_WAVES;
                ci = ni;
                cb = nbx;
                if (t >= T) break;
            }
        }
        __syncthreads();
        for (int r = tid; r < nr * 16; r += RG_THREADS) {
            const int i = r >> 4, row = r & 15;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < RG_WAVES; ++w) v += part[(i * RG_WAVES + w) * 16 + row];
            const int n = (ub + i) * RB + row;
            if (n < N) {
                const float sc = ld_global(reinterpret_cast<const float *>(
                    packed + (size_t)(ub + i) * rb_bytes + (size_t)P * Q8R_TILE_BYTES) + row);
                const float out = sc * (v - 128.f * xsum);
                if (it.out_f32)
                    st_global<float>(it.y, n, out);
                else
                    st_global<uint16_t>(it.y, n, f32_to_bf16(out));
            }
        }
    }
}

// LIST = false: one matrix (`single`, workgroup j takes rowblocks
// [j n / G, (j + 1) n / G)); LIST = true: a device work list of GEMVs
// (workgroup j walks the (matrix, rowblock) range [starts[j], starts[j + 1])).
template <bool LIST>
__global__ void __launch_bounds__(RG_THREADS, 4)
q8row_gemv_kernel(const WorkItem *__restrict__ items, const WorkStart *__restrict__ starts,
                  WorkItem single) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (!LIST) {
        const int64_t G = gridDim.x, j = blockIdx.x, n = single.units;
        const int u0 = (int)(j * n / G), u1 = (int)((j + 1) * n / G);
        if (u0 < u1) rg_range(single, u0, u1, smem, tid, lane, wave);
        return;
    }
    const WorkStart s = starts[blockIdx.x], e = starts[blockIdx.x + 1];
#pragma unroll 1
    for (int i = s.item; i < e.item || (i == e.item && e.unit > 0); ++i) {
        const WorkItem it = items[i];
        const int u0 = (i == s.item) ? s.unit : 0;
        const int u1 = (i == e.item) ? e.unit : it.units;
        if (u0 < u1) rg_range(it, u0, u1, smem, tid, lane, wave);
    }
}

hipError_t launch_q8row_gemv(const uint8_t *packed, const uint16_t *x, void *y, int64_t N,
                             int64_t K, bool out_f32, int cus, hipStream_t s) {
    WorkItem it{};
    it.packed = packed;
    it.x = x;
    it.y = y;
    it.N = (int32_t)N;
    it.K = (int32_t)K;
    it.P = (int32_t)ceil_div(K, Q8R_TILE_K);
    it.units = (int32_t)ceil_div(N, RB);
    it.out_f32 = out_f32 ? 1 : 0;
    const int grid = it.units < cus * 4 ? it.units : cus * 4;
    hipLaunchKernelGGL((q8row_gemv_kernel<false>), dim3(grid), dim3(RG_THREADS), rg_lds_bytes(K),
                       s, (const WorkItem *)nullptr, (const WorkStart *)nullptr, it);
    return hipGetLastError();
}

int q8row_gemv_wgs_per_cu() { return 4; }

hipError_t launch_q8row_gemv_list(const WorkItem *items, const WorkStart *starts, int grid,
                                  int64_t kmax, hipStream_t s) {
    WorkItem none{};
    hipLaunchKernelGGL((q8row_gemv_kernel<true>), dim3(grid), dim3(RG_THREADS), rg_lds_bytes(kmax),
                       s, items, starts, none);
    return hipGetLastError();
}

}  // namespace qg
