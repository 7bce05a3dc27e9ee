// MXFP4 (E2M1 codes, one E8M0 scale per 32) decode GEMV and the routed-expert
// MoE layer for one token (Deltafin / Kimi K3 page, aihot.virxact.com:
// "How it works" -- the router selects the top-16 experts of each layer and
// only those are read; compute list -- fused MXFP4 dequant + GEMV with the
// e8m0 scale applied to the exponent).
//
// Dequantization uses gfx950's v_cvt_scalef32_pk_{bf16,f32}_fp4: two codes of
// one byte (low nibble first) times 2^(e-127), where the scale operand is the
// fp32 whose exponent field is the E8M0 byte.  E2M1 values have at most two
// significant bits, so the scaled value is exact in bf16 and in fp32.
//
// MoE, three launches on one stream, the expert ids never leave the device:
//   A  item = (slot s, rowblock of F): g and u rows of expert ids[s] against
//      x (bf16 in LDS), h = silu(g) * u in fp32 -> workspace h[s][F].
//   B  item = (slot s, rowblock of H): Wdown[ids[s]] rows against h[s]
//      (fp32 in LDS) -> workspace part[s][H].
//   C  y[n] = sum_s w[s] * part[s][n] in slot order (deterministic, no
//      atomics), rounded once; also writes the status word.
#include "qg_internal.h"

namespace qg {

// Dot of one 256-k tile of one row (this lane's share) with bf16 x in LDS.
__device__ __forceinline__ float fp4_tile_dot_bf16(u32x4_t c0, u32x4_t c1, unsigned e0,
                                                   unsigned e1, const uint4 *xp, float acc) {
    // xp points at x[256p + 32kg] as uint4 (8 bf16); half jh adds 16 uint4.
#pragma unroll
    for (int jh = 0; jh < 2; ++jh) {
        const u32x4_t c = jh ? c1 : c0;
        const float sc = e8m0_as_f32(jh ? e1 : e0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 xv = xp[16 * jh + i];
            acc = dot2_bf16(fp4_pair_bf16<0>(c[i], sc), xv.x, acc);
            acc = dot2_bf16(fp4_pair_bf16<1>(c[i], sc), xv.y, acc);
            acc = dot2_bf16(fp4_pair_bf16<2>(c[i], sc), xv.z, acc);
            acc = dot2_bf16(fp4_pair_bf16<3>(c[i], sc), xv.w, acc);
        }
    }
    return acc;
}

// Dot of one 256-k tile with fp32 activations in LDS (the SwiGLU output).
__device__ __forceinline__ float fp4_tile_dot_f32(u32x4_t c0, u32x4_t c1, unsigned e0,
                                                  unsigned e1, const float4 *hp, float acc) {
    // hp points at h[256p + 32kg] as float4; half jh adds 32 float4.
#pragma unroll
    for (int jh = 0; jh < 2; ++jh) {
        const u32x4_t c = jh ? c1 : c0;
        const float sc = e8m0_as_f32(jh ? e1 : e0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 ha = hp[32 * jh + 2 * i], hb = hp[32 * jh + 2 * i + 1];
            f32x2_t v;
            v = fp4_pair_f32<0>(c[i], sc);
            acc = fmaf(v[0], ha.x, acc);
            acc = fmaf(v[1], ha.y, acc);
            v = fp4_pair_f32<1>(c[i], sc);
            acc = fmaf(v[0], ha.z, acc);
            acc = fmaf(v[1], ha.w, acc);
            v = fp4_pair_f32<2>(c[i], sc);
            acc = fmaf(v[0], hb.x, acc);
            acc = fmaf(v[1], hb.y, acc);
            v = fp4_pair_f32<3>(c[i], sc);
            acc = fmaf(v[0], hb.z, acc);
            acc = fmaf(v[1], hb.w, acc);
        }
    }
    return acc;
}

struct Fp4Slot {
    u32x4_t c0, c1;
    unsigned e0, e1;
};

__device__ __forceinline__ Fp4Slot fp4_load(const uint8_t *tb, int lane) {
    Fp4Slot r;
    r.c0 = ld_nt(reinterpret_cast<const u32x4_t *>(tb) + lane);
    r.c1 = ld_nt(reinterpret_cast<const u32x4_t *>(tb + 1024) + lane);
    r.e0 = tb[2048 + lane];
    r.e1 = tb[2048 + 64 + lane];
    return r;
}

// Stage bf16 x [K] into LDS as P*256 elements, zero past K.
__device__ __forceinline__ void stage_x_bf16(uint4 *xl, const uint16_t *x, int K, int P,
                                             int tid, int nthreads) {
    const int nx4 = K / 8;
    for (int i = tid; i < P * 32; i += nthreads) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (i < nx4) v = reinterpret_cast<const uint4 *>(x)[i];
        xl[i] = v;
    }
}

// Sum of this wave's lanes for each of the 16 rows (k-slices kg = lane >> 4).
__device__ __forceinline__ float reduce_kslices(float a) {
    a += __shfl_xor(a, 16);
    a += __shfl_xor(a, 32);
    return a;
}

// ------------------------------------------------------------ single matrix GEMV
template <int WAVES, int TPW>
__global__ void __launch_bounds__(WAVES * 64)
fp4_gemv_kernel(const uint8_t *__restrict__ packed, const uint16_t *__restrict__ x,
                void *__restrict__ y, int N, int K, int P, int nrb, int out_f32) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint4 *xl = reinterpret_cast<uint4 *>(smem);
    float *red = reinterpret_cast<float *>(smem + (size_t)P * 512);
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), kg = lane >> 4;
    stage_x_bf16(xl, x, K, P, tid, WAVES * 64);
    __syncthreads();
    int par = 0;
    for (int rb = blockIdx.x; rb < nrb; rb += gridDim.x) {
        const uint8_t *base = packed + (size_t)rb * P * FP4_TILE_BYTES;
        float acc = 0.f;
        for (int p0 = wave; p0 < P; p0 += WAVES * TPW) {
            Fp4Slot sl[TPW];
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int p = p0 + j * WAVES;
                if (p < P) sl[j] = fp4_load(base + (size_t)p * FP4_TILE_BYTES, lane);
            }
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int p = p0 + j * WAVES;
                if (p < P)
                    acc = fp4_tile_dot_bf16(sl[j].c0, sl[j].c1, sl[j].e0, sl[j].e1,
                                            xl + 32 * p + 4 * kg, acc);
            }
        }
        acc = reduce_kslices(acc);
        if (lane < 16) red[par * WAVES * 16 + wave * 16 + lane] = acc;
        __syncthreads();
        if (wave == 0 && lane < 16) {
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) v += red[par * WAVES * 16 + w * 16 + lane];
            const int row = rb * RB + lane;
            if (row < N) {
                if (out_f32)
                    reinterpret_cast<float *>(y)[row] = v;
                else
                    reinterpret_cast<uint16_t *>(y)[row] = f32_to_bf16(v);
            }
        }
        par ^= 1;
    }
}

hipError_t launch_fp4_gemv(const uint8_t *packed, const uint16_t *x, void *y, int64_t N,
                           int64_t K, bool out_f32, int cus, hipStream_t s) {
    constexpr int WAVES = 4, TPW = 4;
    const int P = (int)ceil_div(K, FP4_TILE_K);
    const int nrb = (int)ceil_div(N, RB);
    const size_t lds = (size_t)P * 512 + 2 * WAVES * 16 * 4;
    const int grid = (int)(nrb < (int64_t)cus * 8 ? nrb : (int64_t)cus * 8);
    hipLaunchKernelGGL((fp4_gemv_kernel<WAVES, TPW>), dim3(grid), dim3(WAVES * 64), lds, s,
                       packed, x, y, (int)N, (int)K, P, nrb, out_f32 ? 1 : 0);
    return hipGetLastError();
}

// ------------------------------------------------------------ MoE phase A
template <int WAVES, int TPW>
__global__ void __launch_bounds__(WAVES * 64)
moe_gate_up_kernel(const uint8_t *__restrict__ pg, const uint8_t *__restrict__ pu,
                   const uint16_t *__restrict__ x, const int32_t *__restrict__ ids, int E,
                   int H, int F, int P, int nrbF, int items, float *__restrict__ h_ws) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint4 *xl = reinterpret_cast<uint4 *>(smem);
    float *red = reinterpret_cast<float *>(smem + (size_t)P * 512);  // [2][2][WAVES][16]
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), kg = lane >> 4;
    stage_x_bf16(xl, x, H, P, tid, WAVES * 64);
    __syncthreads();
    const int per = (items + gridDim.x - 1) / gridDim.x;
    const int i0 = blockIdx.x * per;
    const int i1 = min(items, i0 + per);
    int par = 0;
    for (int it = i0; it < i1; ++it) {
        const int s = it / nrbF, rb = it % nrbF;
        const int e = ids[s];
        if (e < 0 || e >= E) {  // uniform over the workgroup
            if (wave == 0 && lane < 16) h_ws[(size_t)s * F + rb * RB + lane] = 0.f;
            continue;
        }
        const size_t off = ((size_t)e * nrbF + rb) * (size_t)P * FP4_TILE_BYTES;
        const uint8_t *gb = pg + off, *ub = pu + off;
        float ag = 0.f, au = 0.f;
        for (int p0 = wave; p0 < P; p0 += WAVES * TPW) {
            Fp4Slot sg[TPW], su[TPW];
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int p = p0 + j * WAVES;
                if (p < P) {
                    sg[j] = fp4_load(gb + (size_t)p * FP4_TILE_BYTES, lane);
                    su[j] = fp4_load(ub + (size_t)p * FP4_TILE_BYTES, lane);
                }
            }
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int p = p0 + j * WAVES;
                if (p < P) {
                    const uint4 *xp = xl + 32 * p + 4 * kg;
                    ag = fp4_tile_dot_bf16(sg[j].c0, sg[j].c1, sg[j].e0, sg[j].e1, xp, ag);
                    au = fp4_tile_dot_bf16(su[j].c0, su[j].c1, su[j].e0, su[j].e1, xp, au);
                }
            }
        }
        ag = reduce_kslices(ag);
        au = reduce_kslices(au);
        float *rp = red + par * 2 * WAVES * 16;
        if (lane < 16) {
            rp[wave * 16 + lane] = ag;
            rp[WAVES * 16 + wave * 16 + lane] = au;
        }
        __syncthreads();
        if (wave == 0 && lane < 16) {
            float g = 0.f, u = 0.f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) {
                g += rp[w * 16 + lane];
                u += rp[WAVES * 16 + w * 16 + lane];
            }
            h_ws[(size_t)s * F + rb * RB + lane] = g / (1.f + expf(-g)) * u;
        }
        par ^= 1;
    }
}

// ------------------------------------------------------------ MoE phase B
template <int WAVES, int TPW>
__global__ void __launch_bounds__(WAVES * 64)
moe_down_kernel(const uint8_t *__restrict__ pd, const float *__restrict__ h_ws,
                const int32_t *__restrict__ ids, int E, int H, int F, int P, int nrbH,
                int items, float *__restrict__ part) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    float4 *hl = reinterpret_cast<float4 *>(smem);                       // [P*64] float4
    float *red = reinterpret_cast<float *>(smem + (size_t)P * 1024);    // [2][WAVES][16]
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), kg = lane >> 4;
    const int per = (items + gridDim.x - 1) / gridDim.x;
    const int i0 = blockIdx.x * per;
    const int i1 = min(items, i0 + per);
    int cur = -1, par = 0;
    for (int it = i0; it < i1; ++it) {
        const int s = it / nrbH, rb = it % nrbH;
        if (s != cur) {  // uniform: stage h[s] (zero past F)
            __syncthreads();
            const float4 *src = reinterpret_cast<const float4 *>(h_ws + (size_t)s * F);
            for (int i = tid; i < P * 64; i += WAVES * 64)
                hl[i] = (i < F / 4) ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
            __syncthreads();
            cur = s;
        }
        const int e = ids[s];
        if (e < 0 || e >= E) {
            if (wave == 0 && lane < 16) part[(size_t)s * H + rb * RB + lane] = 0.f;
            continue;
        }
        const uint8_t *db = pd + ((size_t)e * nrbH + rb) * (size_t)P * FP4_TILE_BYTES;
        float acc = 0.f;
        for (int p0 = wave; p0 < P; p0 += WAVES * TPW) {
            Fp4Slot sl[TPW];
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int p = p0 + j * WAVES;
                if (p < P) sl[j] = fp4_load(db + (size_t)p * FP4_TILE_BYTES, lane);
            }
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int p = p0 + j * WAVES;
                if (p < P)
                    acc = fp4_tile_dot_f32(sl[j].c0, sl[j].c1, sl[j].e0, sl[j].e1,
                                           hl + 64 * p + 8 * kg, acc);
            }
        }
        acc = reduce_kslices(acc);
        if (lane < 16) red[par * WAVES * 16 + wave * 16 + lane] = acc;
        __syncthreads();
        if (wave == 0 && lane < 16) {
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) v += red[par * WAVES * 16 + w * 16 + lane];
            part[(size_t)s * H + rb * RB + lane] = v;
        }
        par ^= 1;
    }
}

// ------------------------------------------------------------ MoE phase C
__global__ void __launch_bounds__(256)
moe_combine_kernel(const float *__restrict__ part, const int32_t *__restrict__ ids,
                   const float *__restrict__ w, int E, int H, int top_k, void *__restrict__ y,
                   int out_f32, unsigned *__restrict__ status) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n < H) {
        float v = 0.f;
        for (int s = 0; s < top_k; ++s) {
            const int e = ids[s];
            if (e >= 0 && e < E) v = fmaf(w[s], part[(size_t)s * H + n], v);
        }
        if (out_f32)
            reinterpret_cast<float *>(y)[n] = v;
        else
            reinterpret_cast<uint16_t *>(y)[n] = f32_to_bf16(v);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        unsigned bad = 0;
        for (int s = 0; s < top_k; ++s) {
            const int e = ids[s];
            if (e < 0 || e >= E) bad = 1;
        }
        status[0] = bad;
    }
}

hipError_t launch_moe(const uint8_t *pg, const uint8_t *pu, const uint8_t *pd, int64_t E,
                      int64_t H, int64_t F, const uint16_t *x, int top_k, const int32_t *ids,
                      const float *w, uint8_t *workspace, void *y, bool out_f32, int cus,
                      hipStream_t s) {
    constexpr int WAVES = 4, TPW = 4;
    float *h_ws = reinterpret_cast<float *>(workspace);
    float *part = h_ws + (size_t)top_k * F;
    unsigned *status = reinterpret_cast<unsigned *>(part + (size_t)top_k * H);
    if (top_k > 0) {
        const int PH = (int)ceil_div(H, FP4_TILE_K);  // tiles along H (gate/up rows)
        const int nrbF = (int)(F / RB);
        const int itemsA = top_k * nrbF;
        const int gridA = itemsA < cus * 4 ? itemsA : cus * 4;
        const size_t ldsA = (size_t)PH * 512 + 2 * 2 * WAVES * 16 * 4;
        hipLaunchKernelGGL((moe_gate_up_kernel<WAVES, TPW>), dim3(gridA), dim3(WAVES * 64), ldsA,
                           s, pg, pu, x, ids, (int)E, (int)H, (int)F, PH, nrbF, itemsA, h_ws);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        const int PF = (int)ceil_div(F, FP4_TILE_K);  // tiles along F (down rows)
        const int nrbH = (int)(H / RB);
        const int itemsB = top_k * nrbH;
        const int gridB = itemsB < cus * 4 ? itemsB : cus * 4;
        const size_t ldsB = (size_t)PF * 1024 + 2 * WAVES * 16 * 4;
        hipLaunchKernelGGL((moe_down_kernel<WAVES, TPW>), dim3(gridB), dim3(WAVES * 64), ldsB, s,
                           pd, h_ws, ids, (int)E, (int)H, (int)F, PF, nrbH, itemsB, part);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)ceil_div(H, 256)), dim3(256), 0, s,
                       part, ids, w, (int)E, (int)H, top_k, y, out_f32 ? 1 : 0, status);
    return hipGetLastError();
}

}  // namespace qg
