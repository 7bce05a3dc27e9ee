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

__global__ void __launch_bounds__(RG_THREADS, 4)
q8row_gemv_kernel(const uint8_t *__restrict__ packed, const uint16_t *__restrict__ x,
                  void *__restrict__ y, int N, int K, int P, int nrb, int out_f32) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int nb = (P + RG_TPB - 1) / RG_TPB;
    const int KS = nb * RG_TPB * Q8R_TILE_K;  // staged x length (zero past K)
    float *xl = reinterpret_cast<float *>(smem);                  // [KS]
    float *part = xl + KS;                                         // [RMAX][WAVES][16]
    float *red = part + RG_RMAX * RG_WAVES * 16;                   // [THREADS]
    const int tid = threadIdx.x, lane = tid & 63, kg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t G = gridDim.x, j = blockIdx.x;
    const int u0 = (int)(j * nrb / G), u1 = (int)((j + 1) * nrb / G);
    if (u0 >= u1) return;
    const size_t rb_bytes = (size_t)P * Q8R_TILE_BYTES + Q8R_RB_TAIL;
    // stage x as fp32 and take sum_k x: each thread adds its elements in k
    // order, then the threads' sums are added pairwise in a fixed tree
    float own = 0.f;
    for (int k = tid; k < KS; k += RG_THREADS) {
        float v = 0.f;
        if (k < K) v = bf16_lo((unsigned)x[k]);
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
        int t = wave, ci = t / nb, cb = t % nb;
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
                if (out_f32)
                    st_global<float>(y, n, out);
                else
                    st_global<uint16_t>(y, n, f32_to_bf16(out));
            }
        }
    }
}

hipError_t launch_q8row_gemv(const uint8_t *packed, const uint16_t *x, void *y, int64_t N,
                             int64_t K, bool out_f32, int cus, hipStream_t s) {
    const int P = (int)ceil_div(K, Q8R_TILE_K);
    const int nrb = (int)ceil_div(N, RB);
    const int nb = (int)ceil_div(P, RG_TPB);
    const size_t lds = (size_t)nb * RG_TPB * Q8R_TILE_K * 4 + (size_t)RG_RMAX * RG_WAVES * 16 * 4 +
                       (size_t)RG_THREADS * 4;
    const int grid = nrb < cus * 4 ? nrb : cus * 4;
    hipLaunchKernelGGL(q8row_gemv_kernel, dim3(grid), dim3(RG_THREADS), lds, s, packed, x, y,
                       (int)N, (int)K, P, nrb, out_f32 ? 1 : 0);
    return hipGetLastError();
}

}  // namespace qg
