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
//   A  unit = (slot s, rowblock of F): the g and u rows of expert ids[s]
//      against x (bf16 in LDS, multiply-adds on the bf16 MFMA), h = silu(g)
//      * u in fp32 -> workspace h[s][F].
//   B  unit = (slot s, rowblock of H): Wdown[ids[s]] rows against h[s]
//      (fp32 in LDS) -> workspace part[s][H].
//   C  y[n] = sum_s w[s] * part[s][n] in slot order (deterministic, no
//      atomics), rounded once; also writes the status word.
// When h of all slots fits in LDS (128 KB: e.g. top-16 of F = 2048), B and C
// are one launch that computes whole rowblocks of y (see below).
// A and B give each workgroup a contiguous range of units and stream them
// like the Q4 decode GEMV: a unit's tiles are cut into batches of 4, every
// fourth batch goes to the same wave, and each wave streams its batches
// double-buffered with the load of each tile of its next batch issued just
// before the arithmetic of the same tile of the current one.  A wave folds
// its sums of a unit into its own LDS slot; the workgroup adds the wave slots
// in wave order when a block of up to 32 units ends.
#include "fp4_stream.h"

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

// One 256-k tile of 16 rows against bf16 x on the MFMA, for a single token:
// the decoded weights are the B operand exactly as loaded (lane l: row l & 15,
// k-slice l >> 4; its dword i of half j is the k-group of 8 at 128j + 32(l >>
// 4) + 8i), and every row of the A operand is x (each lane reads the 8
// values of x that match its own k-group, as the lanes of one k-slice share
// them, one broadcast LDS read).  The k-groups of the four slices fill the
// MFMA's 32 k in a fixed order, the same for both operands, so every element
// of C holds the dot product of row n = lane & 15 (the 16 rows of C are the
// same sum); the caller takes C[0] of lanes 0..15.  Per tile: 32 conversions
// and 8 MFMAs instead of 32 conversions and 32 two-element dot products.
__device__ __forceinline__ f32x4_t fp4_tile_mfma_bf16(u32x4_t c0, u32x4_t c1, unsigned e0,
                                                      unsigned e1, const uint4 *xp, f32x4_t C) {
#pragma unroll
    for (int jh = 0; jh < 2; ++jh) {
        const u32x4_t c = jh ? c1 : c0;
        const float sc = e8m0_as_f32(jh ? e1 : e0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4_t w = {fp4_pair_bf16<0>(c[i], sc), fp4_pair_bf16<1>(c[i], sc),
                               fp4_pair_bf16<2>(c[i], sc), fp4_pair_bf16<3>(c[i], sc)};
            const uint4 xv = xp[16 * jh + i];
            const u32x4_t xa = {xv.x, xv.y, xv.z, xv.w};
            C = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa),
                                                        __builtin_bit_cast(bf16x8_t, w), C, 0,
                                                        0, 0);
        }
    }
    return C;
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

// Fill n 16-byte chunks of LDS, chunk i taken from src(i) (a global load, or
// zero).  Each thread issues the loads of U chunks before it writes any of
// them, so a fill costs about n / (U * nthreads) memory round trips rather
// than one per chunk.
template <int U, typename Src>
__device__ __forceinline__ void lds_fill16(uint4 *dst, int n, int tid, int nthreads, Src src) {
    for (int i0 = tid; i0 < n; i0 += U * nthreads) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * nthreads;
            v[u] = i < n ? src(i) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * nthreads;
            if (i < n) dst[i] = v[u];
        }
    }
}

// Stage bf16 x [K] into LDS as P*256 elements, zero past K.
__device__ __forceinline__ void stage_x_bf16(uint4 *xl, const uint16_t *x, int K, int P,
                                             int tid, int nthreads) {
    const int nx4 = K / 8;
    const uint4 *src = reinterpret_cast<const uint4 *>(x);
    lds_fill16<4>(xl, P * 32, tid, nthreads, [=](int i) {
        return i < nx4 ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    });
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
                    st_global<float>(y, row, v);
                else
                    st_global<uint16_t>(y, row, f32_to_bf16(v));
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

// ------------------------------------------------------------ MoE streaming
constexpr int MS_WAVES = 4;
constexpr int MS_THREADS = MS_WAVES * 64;
constexpr int MS_RMAX = 32;   // units per output block

// Position in a wave's batch stream: unit i (relative to the block), batch b.
struct MsCursor {
    int i, b;
};
__device__ __forceinline__ MsCursor ms_advance(MsCursor c, int nbu) {
    c.b += MS_WAVES;
    while (c.b >= nbu) {  // uniform
        c.b -= nbu;
        ++c.i;
    }
    return c;
}

// ------------------------------------------------------------ MoE phase A
// Units u = s * nrbF + rb; a unit has 2 * nb batches: nb of the gate rows,
// then nb of the up rows (nb = batches of PH tiles).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t moe_a_rsrc(
    const uint8_t *pg, const uint8_t *pu, const int32_t *ids, int E, int nrbF, int PH, int nb,
    int unit, int b, bool valid) {
    // past the wave's last batch the unit may lie past the last slot: no
    // id is read for it
    const int s = valid ? unit / nrbF : 0, rb = valid ? unit - s * nrbF : 0;
    const int e = valid ? ids[s] : -1;
    const bool ok = valid && e >= 0 && e < E;
    const uint8_t *mat = (b < nb) ? pg : pu;
    const uint8_t *base = mat + ((size_t)(ok ? e : 0) * nrbF + rb) * (size_t)PH * FP4_TILE_BYTES;
    return make_rsrc(uniform_ptr(base), ok ? (unsigned)PH * FP4_TILE_BYTES : 0u);
}

__global__ void __launch_bounds__(MS_THREADS, 4)
moe_gate_up_kernel(const uint8_t *__restrict__ pg, const uint8_t *__restrict__ pu,
                   const uint16_t *__restrict__ x, const int32_t *__restrict__ ids, int E,
                   int H, int F, int PH, int nrbF, int units, float *__restrict__ h_ws) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int nb = (PH + MS_TPB - 1) / MS_TPB, nbu = 2 * nb;
    uint4 *xl = reinterpret_cast<uint4 *>(smem);                               // [nb*4 tiles][32]
    float *part = reinterpret_cast<float *>(smem + (size_t)nb * MS_TPB * 512);  // [RMAX][WAVES][2][16]
    const int tid = threadIdx.x, lane = tid & 63, kg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t G = gridDim.x, j = blockIdx.x;
    const int u0 = (int)(j * units / G), u1 = (int)((j + 1) * units / G);
    if (u0 >= u1) return;
#pragma unroll 1
    for (int ub = u0; ub < u1; ub += MS_RMAX) {
        const int nr = min(u1 - ub, MS_RMAX);
        const int T = nr * nbu;
        int t = (wave - (ub & 3) * (nbu & 3)) & 3;  // absolute batch index = wave mod 4
        MsCursor ca = {t / nbu, t % nbu};
        Fp4Batch A, B;
        f32x4_t C = {0.f, 0.f, 0.f, 0.f};
        {
            // the first batch loads while x is staged and the sums cleared
            const __amdgpu_buffer_rsrc_t rs =
                moe_a_rsrc(pg, pu, ids, E, nrbF, PH, nb, ub + ca.i, ca.b, t < T);
            const int tb = (ca.b % nb) * MS_TPB;
#pragma unroll
            for (int q = 0; q < MS_TPB; ++q) fp4_tile_load(A, q, rs, tb + q, PH, lane);
        }
        if (ub == u0) stage_x_bf16(xl, x, H, nb * MS_TPB, tid, MS_THREADS);
        for (int i = tid; i < nr * MS_WAVES * 32; i += MS_THREADS) part[i] = 0.f;
        __syncthreads();  // x staged, partial sums cleared
#pragma unroll 1
        for (;;) {
            if (t >= T) break;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                Fp4Batch &Cur = half ? B : A;
                Fp4Batch &Nxt = half ? A : B;
                const MsCursor cn = ms_advance(ca, nbu);
                const bool nvalid = t + MS_WAVES < T;
                const __amdgpu_buffer_rsrc_t rs =
                    moe_a_rsrc(pg, pu, ids, E, nrbF, PH, nb, ub + cn.i, cn.b, nvalid);
                const int tbn = (cn.b % nb) * MS_TPB, tbc = (ca.b % nb) * MS_TPB;
#pragma unroll
                for (int q = 0; q < MS_TPB; ++q) {
                    __builtin_amdgcn_sched_barrier(0);
                    fp4_tile_load(Nxt, q, rs, tbn + q, PH, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    C = fp4_tile_mfma_bf16(Cur.c0[q], Cur.c1[q], Cur.e0[q], Cur.e1[q],
                                           xl + 32 * (tbc + q) + 4 * kg, C);
                }
                // flush at the wave's last batch of this unit's gate or up rows
                const bool gate = ca.b < nb;
                const bool last = !nvalid || cn.i != ca.i || (gate && cn.b >= nb);
                if (last) {
                    if (lane < 16)
                        part[((ca.i * MS_WAVES + wave) * 2 + (gate ? 0 : 1)) * 16 + lane] += C[0];
                    C = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
                t += MS_WAVES;
                ca = cn;
                if (t >= T) break;
            }
        }
        __syncthreads();
        for (int r = tid; r < nr * 16; r += MS_THREADS) {
            const int i = r >> 4, row = r & 15;
            float g = 0.f, u = 0.f;
#pragma unroll
            for (int w = 0; w < MS_WAVES; ++w) {
                g += part[((i * MS_WAVES + w) * 2 + 0) * 16 + row];
                u += part[((i * MS_WAVES + w) * 2 + 1) * 16 + row];
            }
            const int unit = ub + i, s = unit / nrbF, rb = unit - s * nrbF;
            h_ws[(size_t)s * F + rb * RB + row] = g / (1.f + expf(-g)) * u;
        }
        __syncthreads();  // part is reused by the next block
    }
}

// ------------------------------------------------------------ MoE phase B
// Units u = s * nrbH + rb; h[s] is staged per run of units of one slot.
__global__ void __launch_bounds__(MS_THREADS, 4)
moe_down_kernel(const uint8_t *__restrict__ pd, const float *__restrict__ h_ws,
                const int32_t *__restrict__ ids, int E, int H, int F, int PF, int nrbH,
                int units, float *__restrict__ part_ws) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int nb = (PF + MS_TPB - 1) / MS_TPB;
    float4 *hl = reinterpret_cast<float4 *>(smem);                               // [nb*4 tiles][64]
    float *part = reinterpret_cast<float *>(smem + (size_t)nb * MS_TPB * 1024);  // [RMAX][WAVES][16]
    const int tid = threadIdx.x, lane = tid & 63, kg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t G = gridDim.x, j = blockIdx.x;
    const int u0 = (int)(j * units / G), u1 = (int)((j + 1) * units / G);
#pragma unroll 1
    for (int ub = u0; ub < u1;) {
        const int s = ub / nrbH;
        const int e = ids[s];
        const bool ok = e >= 0 && e < E;
        const int nr = min(min(u1, (s + 1) * nrbH) - ub, MS_RMAX);  // one slot per block
        const int rb0 = ub - s * nrbH;
        const int T = nr * nb;
        int t = (wave - (ub & 3) * (nb & 3)) & 3;
        MsCursor ca = {t / nb, t % nb};
        const uint8_t *ebase = pd + (size_t)(ok ? e : 0) * nrbH * (size_t)PF * FP4_TILE_BYTES;
        Fp4Batch A, B;
        float acc = 0.f;
        {
            // the first batch loads while h[s] is staged
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(
                uniform_ptr(ebase + (size_t)(rb0 + ca.i) * PF * FP4_TILE_BYTES),
                (ok && t < T) ? (unsigned)PF * FP4_TILE_BYTES : 0u);
#pragma unroll
            for (int q = 0; q < MS_TPB; ++q) fp4_tile_load(A, q, rs, ca.b * MS_TPB + q, PF, lane);
        }
        __syncthreads();  // the previous block is written out
        {
            const uint4 *src = reinterpret_cast<const uint4 *>(h_ws + (size_t)s * F);
            const int nh4 = F / 4;
            lds_fill16<4>(reinterpret_cast<uint4 *>(hl), nb * MS_TPB * 64, tid, MS_THREADS,
                          [=](int i) { return i < nh4 ? src[i] : make_uint4(0u, 0u, 0u, 0u); });
            for (int i = tid; i < nr * MS_WAVES * 16; i += MS_THREADS) part[i] = 0.f;
        }
        __syncthreads();
#pragma unroll 1
        for (;;) {
            if (t >= T) break;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                Fp4Batch &Cur = half ? B : A;
                Fp4Batch &Nxt = half ? A : B;
                const MsCursor cn = ms_advance(ca, nb);
                const bool nvalid = t + MS_WAVES < T;
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(
                    uniform_ptr(ebase + (size_t)(rb0 + cn.i) * PF * FP4_TILE_BYTES),
                    (ok && nvalid) ? (unsigned)PF * FP4_TILE_BYTES : 0u);
#pragma unroll
                for (int q = 0; q < MS_TPB; ++q) {
                    __builtin_amdgcn_sched_barrier(0);
                    fp4_tile_load(Nxt, q, rs, cn.b * MS_TPB + q, PF, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    acc = fp4_tile_dot_f32(Cur.c0[q], Cur.c1[q], Cur.e0[q], Cur.e1[q],
                                           hl + 64 * (ca.b * MS_TPB + q) + 8 * kg, acc);
                }
                if (!nvalid || cn.i != ca.i) {
                    acc = reduce_kslices(acc);
                    if (lane < 16) part[(ca.i * MS_WAVES + wave) * 16 + lane] += acc;
                    acc = 0.f;
                }
                t += MS_WAVES;
                ca = cn;
                if (t >= T) break;
            }
        }
        __syncthreads();
        for (int r = tid; r < nr * 16; r += MS_THREADS) {
            const int i = r >> 4, row = r & 15;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < MS_WAVES; ++w) v += part[(i * MS_WAVES + w) * 16 + row];
            part_ws[(size_t)s * H + (rb0 + i) * RB + row] = v;
        }
        ub += nr;
    }
}

// ------------------------------------------------------------ MoE phase B+C fused
// When h of every slot fits in LDS (top_k * F <= MF_HMAX floats), one
// workgroup of 16 waves per CU stages all of them once and computes whole
// output rowblocks of y: unit = rowblock rb of H, its batches (slot s, 4 tiles
// of F) go to the waves in turn, each wave sums w_s * (its batches' dot
// products), and the 16 wave sums are added in wave order (deterministic).
// This replaces the per-slot partials and the combine launch.
constexpr int MF_WAVES = 16;
constexpr int MF_THREADS = MF_WAVES * 64;
constexpr int MF_HMAX = 32768;  // fp32 values of h staged (128 KB)
constexpr int MF_UMAX = 8;      // units whose wave sums are added together

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mf_rsrc(const uint8_t *pd, const int32_t *ids,
                                                          int E, int nrbH, int PF, int rb, int s,
                                                          bool valid) {
    const int e = valid ? ids[s] : -1;
    const bool ok = valid && e >= 0 && e < E;
    const uint8_t *base = pd + ((size_t)(ok ? e : 0) * nrbH + rb) * (size_t)PF * FP4_TILE_BYTES;
    return make_rsrc(uniform_ptr(base), ok ? (unsigned)PF * FP4_TILE_BYTES : 0u);
}

__global__ void __launch_bounds__(MF_THREADS, 1)
moe_down_fused_kernel(const uint8_t *__restrict__ pd, const float *__restrict__ h_ws,
                      const int32_t *__restrict__ ids, const float *__restrict__ w, int E, int H,
                      int F, int PF, int nrbH, int top_k, void *__restrict__ y, int out_f32,
                      unsigned *__restrict__ status) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int nb = (PF + MS_TPB - 1) / MS_TPB;       // batches per slot
    const int hstride = nb * MS_TPB * 64;             // float4 per staged slot
    float4 *hl = reinterpret_cast<float4 *>(smem);
    float *red = reinterpret_cast<float *>(smem + (size_t)top_k * hstride * 16);  // [UMAX][WAVES][16]
    float *wl = red + MF_UMAX * MF_WAVES * 16;                                      // [top_k]
    const int tid = threadIdx.x, lane = tid & 63, kg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (blockIdx.x == 0 && tid == 0) {
        unsigned bad = 0;
        for (int s = 0; s < top_k; ++s)
            if (ids[s] < 0 || ids[s] >= E) bad = 1;
        status[0] = bad;
    }
    const int T = top_k * nb;  // batches per unit
    const int G = gridDim.x;
    const MsCursor first = {wave / nb, wave % nb};  // a wave's first batch of every unit
    Fp4Batch A, B;
    int rb = blockIdx.x;
    int rb0 = rb, ui = 0;  // first unit of the pending slots, and their count
    {
        const __amdgpu_buffer_rsrc_t rs = mf_rsrc(pd, ids, E, nrbH, PF, rb, first.i, wave < T);
#pragma unroll
        for (int q = 0; q < MS_TPB; ++q) fp4_tile_load(A, q, rs, first.b * MS_TPB + q, PF, lane);
    }
    // while the first batch loads: stage every slot's h and weight
    for (int i = tid; i < top_k; i += MF_THREADS) {
        const int e = ids[i];
        wl[i] = (e >= 0 && e < E) ? w[i] : 0.f;  // an invalid id contributes nothing
    }
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(h_ws);
        const int nh4 = F / 4;
        lds_fill16<8>(reinterpret_cast<uint4 *>(hl), top_k * hstride, tid, MF_THREADS,
                      [=](int i) {
                          const int s = i / hstride, c = i - s * hstride;
                          return c < nh4 ? src[(size_t)s * nh4 + c] : make_uint4(0u, 0u, 0u, 0u);
                      });
    }
    __syncthreads();
#pragma unroll 1
    for (;;) {
        // this unit's first batch is in A; the last step of the unit already
        // loads the next unit's first batch
        int t = wave, steps = 0;
        MsCursor ca = first;
        float acc = 0.f;
#pragma unroll 1
        for (;;) {
            if (t >= T) break;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                Fp4Batch &Cur = half ? B : A;
                Fp4Batch &Nxt = half ? A : B;
                MsCursor cn = ca;
                cn.b += MF_WAVES;
                while (cn.b >= nb) {  // uniform
                    cn.b -= nb;
                    ++cn.i;
                }
                const bool more = t + MF_WAVES < T;
                const int nrb = more ? rb : rb + G;
                if (!more) cn = first;
                const bool nvalid = more || (nrb < nrbH && wave < T);
                const __amdgpu_buffer_rsrc_t rs = mf_rsrc(pd, ids, E, nrbH, PF, nrb, cn.i, nvalid);
                const float4 *hs = hl + ca.i * hstride;
                float bs = 0.f;
#pragma unroll
                for (int q = 0; q < MS_TPB; ++q) {
                    __builtin_amdgcn_sched_barrier(0);
                    fp4_tile_load(Nxt, q, rs, cn.b * MS_TPB + q, PF, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    bs = fp4_tile_dot_f32(Cur.c0[q], Cur.c1[q], Cur.e0[q], Cur.e1[q],
                                          hs + 64 * (ca.b * MS_TPB + q) + 8 * kg, bs);
                }
                acc = fmaf(wl[ca.i], bs, acc);
                ++steps;
                t += MF_WAVES;
                ca = cn;
                if (t >= T) break;
            }
        }
        // the wave's sums of this unit wait in the unit's own slot; a wave
        // goes on to its next unit without waiting for the others, and the
        // workgroup adds the slots of up to MF_UMAX units at once
        acc = reduce_kslices(acc);
        if (lane < 16) red[(ui * MF_WAVES + wave) * 16 + lane] = acc;
        ++ui;
        const int rbn = rb + G;
        if (ui == MF_UMAX || rbn >= nrbH) {
            __syncthreads();
            for (int r = tid; r < ui * 16; r += MF_THREADS) {
                const int i = r >> 4, row = r & 15;
                float v = 0.f;
#pragma unroll
                for (int wv = 0; wv < MF_WAVES; ++wv) v += red[(i * MF_WAVES + wv) * 16 + row];
                const int n = (rb0 + i * G) * RB + row;
                if (out_f32)
                    st_global<float>(y, n, v);
                else
                    st_global<uint16_t>(y, n, f32_to_bf16(v));
            }
            __syncthreads();  // the slots are reused by the next units
            ui = 0;
            rb0 = rbn;
        }
        rb = rbn;
        if (rb >= nrbH) break;
        if (steps & 1) A = B;  // the next unit's first batch went to B
    }
}

// ------------------------------------------------------------ MoE phase C
// y[t][n] = sum_s w[t][s] * part[t][s][n] in slot order for the position t =
// blockIdx.y (one position for the single-token layer).  status (when not
// null) receives 1 if any id of position 0 was out of range.
__global__ void __launch_bounds__(256)
moe_combine_kernel(const float *__restrict__ part, const int32_t *__restrict__ ids,
                   const float *__restrict__ w, int E, int H, int top_k, void *__restrict__ y,
                   int out_f32, unsigned *__restrict__ status) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    const int t = blockIdx.y;
    part += (size_t)t * top_k * H;
    ids += (size_t)t * top_k;
    w += (size_t)t * top_k;
    constexpr int C = 16;  // slots whose loads are issued together
    float v = 0.f;
    unsigned bad = 0;
#pragma unroll 1
    for (int s0 = 0; s0 < top_k; s0 += C) {
        float pv[C], wv[C];
        int ev[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int s = s0 + c;
            ev[c] = s < top_k ? ids[s] : 0;
            wv[c] = s < top_k ? w[s] : 0.f;
            pv[c] = (s < top_k && n < H) ? part[(size_t)s * H + n] : 0.f;
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if (s0 + c < top_k) {
                if (ev[c] >= 0 && ev[c] < E) v = fmaf(wv[c], pv[c], v);
                else bad = 1;
            }
        }
    }
    if (n < H) {
        const size_t o = (size_t)t * H + n;
        if (out_f32)
            st_global<float>(y, o, v);
        else
            st_global<uint16_t>(y, o, f32_to_bf16(v));
    }
    if (status && t == 0 && blockIdx.x == 0 && threadIdx.x == 0) status[0] = bad;
}

hipError_t launch_moe_combine(const float *part, const int32_t *ids, const float *w, int64_t E,
                              int64_t H, int top_k, int T, void *y, bool out_f32,
                              unsigned *status, hipStream_t s) {
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)ceil_div(H, 256), (unsigned)T),
                       dim3(256), 0, s, part, ids, w, (int)E, (int)H, top_k, y,
                       out_f32 ? 1 : 0, status);
    return hipGetLastError();
}

hipError_t launch_moe(const uint8_t *pg, const uint8_t *pu, const uint8_t *pd, int64_t E,
                      int64_t H, int64_t F, const uint16_t *x, int top_k, const int32_t *ids,
                      const float *w, uint8_t *workspace, void *y, bool out_f32, int cus,
                      hipStream_t s, unsigned *status_out) {
    float *h_ws = reinterpret_cast<float *>(workspace);
    float *part = h_ws + (size_t)top_k * F;
    unsigned *status =
        status_out ? status_out : reinterpret_cast<unsigned *>(part + (size_t)top_k * H);
    if (top_k > 0) {
        const int PH = (int)ceil_div(H, FP4_TILE_K);  // tiles along H (gate/up rows)
        const int nrbF = (int)(F / RB);
        const int unitsA = top_k * nrbF;
        const int gridA = unitsA < cus * 4 ? unitsA : cus * 4;
        const size_t ldsA = (size_t)ceil_div(PH, MS_TPB) * MS_TPB * 512 +
                            (size_t)MS_RMAX * MS_WAVES * 2 * 16 * 4;
        hipLaunchKernelGGL(moe_gate_up_kernel, dim3(gridA), dim3(MS_THREADS), ldsA, s, pg, pu, x,
                           ids, (int)E, (int)H, (int)F, PH, nrbF, unitsA, h_ws);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        const int PF = (int)ceil_div(F, FP4_TILE_K);  // tiles along F (down rows)
        const int nrbH = (int)(H / RB);
        const int64_t hstaged = (int64_t)top_k * ceil_div(PF, MS_TPB) * MS_TPB * 256;
        if (hstaged <= MF_HMAX) {
            // down projection and the weighted sum over slots in one launch
            const int gridF = nrbH < cus ? nrbH : cus;
            const size_t ldsF = (size_t)hstaged * 4 + (size_t)MF_UMAX * MF_WAVES * 16 * 4 +
                                (size_t)top_k * 4;
            hipLaunchKernelGGL(moe_down_fused_kernel, dim3(gridF), dim3(MF_THREADS), ldsF, s, pd,
                               h_ws, ids, w, (int)E, (int)H, (int)F, PF, nrbH, top_k, y,
                               out_f32 ? 1 : 0, status);
            return hipGetLastError();
        }
        const int unitsB = top_k * nrbH;
        const int gridB = unitsB < cus * 4 ? unitsB : cus * 4;
        const size_t ldsB = (size_t)ceil_div(PF, MS_TPB) * MS_TPB * 1024 +
                            (size_t)MS_RMAX * MS_WAVES * 16 * 4;
        hipLaunchKernelGGL(moe_down_kernel, dim3(gridB), dim3(MS_THREADS), ldsB, s, pd, h_ws, ids,
                           (int)E, (int)H, (int)F, PF, nrbH, unitsB, part);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return launch_moe_combine(part, ids, w, E, H, top_k, 1, y, out_f32, status, s);
}

}  // namespace qg
