// MXFP4 routed experts for T positions in one pass (T = 1..32): the
// verification pass of a speculative decoder sends every draft position
// through each MoE layer, and each position has its own router choice
// (Deltafin / Kimi K3 page, aihot.virxact.com, "How it works": the router
// picks the top-k experts of a token and only those are read).  Here an
// expert chosen by several positions is read once for all of them, so a
// pass reads the union of the positions' experts instead of T * top_k
// experts.
//
// Four launches on one stream; the ids never leave the device:
//   R  one workgroup groups the valid (position t, slot s) pairs, p = t *
//      top_k + s, by expert id: groups of at most mc pairs of one expert,
//      ordered by expert id and then by p, written as records
//      {e, c, p_0 .. p_{c-1}} with their count.
//   A  unit = (group, rowblock of F): the gate and up rows of the group's
//      expert against the c positions' x (bf16 in LDS) -> h[p] = silu(g) u,
//      fp32, in the workspace.
//   B  unit = (group, rowblock of H): the down rows against the c pairs' h
//      -> part[p], fp32, in the workspace.
//   C  y[t] = sum_s w[t][s] part[t top_k + s] in slot order (the combine of
//      the single-token layer, one position per grid row).
// A and B multiply on the matrix cores.  A tile's lane holds 32 consecutive
// codes of row l & 15 per half (k = 128j + 32(l >> 4) + ...), i.e. four
// 8-k pieces; each piece, through the exact scaled FP4 convert, is the bf16x8
// B operand of one v_mfma_f32_16x16x32_bf16, whose A operand is the same k of
// the group's activation rows (rows past c are zero).  The contraction over a
// tile thus takes the k of each MFMA in a different (consistent) order than
// the VALU kernels, which rounding aside gives the same sums.  h is fp32;
// B splits it into bf16 hi + lo (|h - hi - lo| <= 2^-16 |h|) and multiplies
// both, so its error stays far below a bf16 output's.
// Within a unit a wave adds its batches (4 tiles of one rowblock, every 4th
// batch of the unit) in K order and the workgroup adds the four waves' sums
// in wave order, so results are deterministic.
#include "fp4_stream.h"

namespace qg {

constexpr int MT_WAVES = 4;
constexpr int MT_THREADS = MT_WAVES * 64;
constexpr int MT_RMAX = 8;          // units per block
constexpr int MT_GREC = 8;          // int32 per group record: e, c, p[4], 0, 0
constexpr int MT_ROUTE_THREADS = 1024;

struct MtCursor {
    int i, b;  // unit within the block, batch within the unit
};
__device__ __forceinline__ MtCursor mt_advance(MtCursor c, int nbu) {
    c.b += MT_WAVES;
    while (c.b >= nbu) {  // uniform
        c.b -= nbu;
        ++c.i;
    }
    return c;
}

// ------------------------------------------------------------ R: routing
// key = expert id of a valid pair, -1 otherwise.  rank = valid pairs of the
// same expert before it; a pair whose rank is a multiple of mc starts a
// group, and the group index of a pair is the number of group starts of
// smaller expert ids plus rank / mc.
__global__ void __launch_bounds__(MT_ROUTE_THREADS)
moe_route_kernel(const int32_t *__restrict__ ids, int P, int E, int mc,
                 int32_t *__restrict__ groups, unsigned *__restrict__ hdr) {
    __shared__ int key[MOE_PAIRS_MAX], rank[MOE_PAIRS_MAX], start[MOE_PAIRS_MAX];
    __shared__ unsigned s_bad, s_ng;
    const int tid = threadIdx.x;
    if (tid == 0) {
        s_bad = 0;
        s_ng = 0;
    }
    for (int p = tid; p < P; p += MT_ROUTE_THREADS) {
        const int e = ids[p];
        key[p] = (e >= 0 && e < E) ? e : -1;
    }
    __syncthreads();
    for (int p = tid; p < P; p += MT_ROUTE_THREADS) {
        const int kp = key[p];
        int r = 0;
        if (kp >= 0) {
            for (int q = 0; q < p; ++q) r += key[q] == kp;
        } else {
            atomicOr(&s_bad, 1u);
        }
        rank[p] = r;
        start[p] = (kp >= 0 && r % mc == 0) ? kp : -1;
    }
    __syncthreads();
    for (int p = tid; p < P; p += MT_ROUTE_THREADS) {
        const int kp = key[p];
        if (kp < 0) continue;
        int before = 0, n = 0;
        for (int q = 0; q < P; ++q) {
            const int sq = start[q];
            before += (sq >= 0) & (sq < kp);
            n += key[q] == kp;
        }
        const int r = rank[p], gid = before + r / mc, slot = r % mc;
        int32_t *g = groups + (size_t)gid * MT_GREC;
        st_global<int32_t>(g, 2 + slot, p);
        if (slot == 0) {
            const int c = min(mc, n - r);
            st_global<int32_t>(g, 0, kp);
            st_global<int32_t>(g, 1, c);
            for (int j = 2 + c; j < MT_GREC; ++j) st_global<int32_t>(g, j, 0);
            atomicAdd(&s_ng, 1u);
        }
    }
    __syncthreads();
    if (tid == 0) {
        st_global<unsigned>(hdr, 0, s_bad);
        st_global<unsigned>(hdr, 1, s_ng);
    }
}

// ------------------------------------------------------------ MFMA tiles
__device__ __forceinline__ bf16x8_t fp4_word_bf16x8(unsigned w, float sc) {
    const u32x4_t v = {fp4_pair_bf16<0>(w, sc), fp4_pair_bf16<1>(w, sc),
                       fp4_pair_bf16<2>(w, sc), fp4_pair_bf16<3>(w, sc)};
    return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ bf16x8_t lds_row8(const uint16_t *p, bool act) {
    bf16x8_t a = {};
    if (act) a = *reinterpret_cast<const bf16x8_t *>(p);
    return a;
}

// One tile (index tp of the staged rows) against one bf16 activation row per
// lane: arow = row (lane & 15) + 32 (lane >> 4); act = the row is one of the
// group's.  Half 0 accumulates into D0, half 1 into D1.
__device__ __forceinline__ void mt_tile_x(u32x4_t c0, u32x4_t c1, unsigned e0, unsigned e1,
                                          const uint16_t *arow, bool act, int tp, f32x4_t &D0,
                                          f32x4_t &D1) {
    const float s0 = e8m0_as_f32(e0), s1 = e8m0_as_f32(e1);
    const uint16_t *a = arow + 256 * tp;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        D0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_row8(a + 8 * i, act),
                                                     fp4_word_bf16x8(c0[i], s0), D0, 0, 0, 0);
        D1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_row8(a + 128 + 8 * i, act),
                                                     fp4_word_bf16x8(c1[i], s1), D1, 0, 0, 0);
    }
}

// The same against split fp32 rows: ahi / alo = the hi and lo bf16 rows.
// hi products go to D0, lo products to D1.
__device__ __forceinline__ void mt_tile_h(u32x4_t c0, u32x4_t c1, unsigned e0, unsigned e1,
                                          const uint16_t *ahi, const uint16_t *alo, bool act,
                                          int tp, f32x4_t &D0, f32x4_t &D1) {
    const float s0 = e8m0_as_f32(e0), s1 = e8m0_as_f32(e1);
    const int o = 256 * tp;
#pragma unroll
    for (int jh = 0; jh < 2; ++jh) {
        const u32x4_t c = jh ? c1 : c0;
        const float sc = jh ? s1 : s0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x8_t B = fp4_word_bf16x8(c[i], sc);
            const int k = o + 128 * jh + 8 * i;
            D0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_row8(ahi + k, act), B, D0, 0, 0, 0);
            D1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_row8(alo + k, act), B, D1, 0, 0, 0);
        }
    }
}

// Group record g: expert id and pair count (wave-uniform).
__device__ __forceinline__ int2 mt_group(const int32_t *groups, int g) {
    const int e = __builtin_amdgcn_readfirstlane(ld_global(groups + (size_t)g * MT_GREC));
    const int c = __builtin_amdgcn_readfirstlane(ld_global(groups + (size_t)g * MT_GREC + 1));
    return make_int2(e, c);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mt_rsrc(const uint8_t *mat, int e, int nrb,
                                                          int rb, int pn, bool valid) {
    const uint8_t *base = mat + ((size_t)e * nrb + rb) * (size_t)pn * FP4_TILE_BYTES;
    return make_rsrc(uniform_ptr(base), valid ? (unsigned)pn * FP4_TILE_BYTES : 0u);
}

__device__ __forceinline__ void mt_flush(float *slot, const f32x4_t &D0, const f32x4_t &D1,
                                         int lane) {
    // lanes 0..15 hold activation rows 0..3 of output row (lane & 15)
    if (lane < 16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) slot[16 * e + lane] += D0[e] + D1[e];
    }
}

// ------------------------------------------------------------ A: gate / up
// Units u = g * nrbF + rb; a unit has 2 * nb batches: nb of the gate rows,
// then nb of the up rows.  Blocks of at most MT_RMAX units never span two
// groups; x is restaged when the group changes.
__global__ void __launch_bounds__(MT_THREADS, 2)
moe_t_gate_up_kernel(const uint8_t *__restrict__ pg, const uint8_t *__restrict__ pu,
                     const uint16_t *__restrict__ X, int top_k, int H, int F, int PH, int nrbF,
                     int mc, const int32_t *__restrict__ groups, const unsigned *__restrict__ hdr,
                     float *__restrict__ h_ws) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int nb = (PH + MS_TPB - 1) / MS_TPB, nbu = 2 * nb;
    const int XS = nb * MS_TPB * 256 + 8;  // row stride (bf16), 16-byte pad
    uint16_t *xl = reinterpret_cast<uint16_t *>(smem);                              // [mc][XS]
    float *part = reinterpret_cast<float *>(smem + (size_t)mc * XS * 2);           // [RMAX][W][2][64]
    const int tid = threadIdx.x, lane = tid & 63, kg = lane >> 4, m = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ng = __builtin_amdgcn_readfirstlane(ld_global(hdr + 1));
    const int64_t units = (int64_t)ng * nrbF, G = gridDim.x, j = blockIdx.x;
    const int u0 = (int)(j * units / G), u1 = (int)((j + 1) * units / G);
    int staged = -1;
#pragma unroll 1
    for (int ub = u0; ub < u1;) {
        const int g = ub / nrbF, rb0 = ub - g * nrbF;
        const int nr = min(min(u1 - ub, nrbF - rb0), MT_RMAX);
        const int2 gr = mt_group(groups, g);
        const int e = gr.x, c = gr.y;
        const int T = nr * nbu;
        int t = wave;
        MtCursor ca = {t / nbu, t % nbu};
        Fp4Batch A, B;
        f32x4_t D0 = {0.f, 0.f, 0.f, 0.f}, D1 = D0;
        {
            // the block's first batch loads while x is staged
            const __amdgpu_buffer_rsrc_t rs =
                mt_rsrc(ca.b < nb ? pg : pu, e, nrbF, rb0 + ca.i, PH, t < T);
            const int tb = (ca.b % nb) * MS_TPB;
#pragma unroll
            for (int q = 0; q < MS_TPB; ++q) fp4_tile_load(A, q, rs, tb + q, PH, lane);
        }
        __syncthreads();  // the previous block is done with x and part
        if (g != staged) {
            const int per = XS / 8;  // 16-byte chunks per staged row (the pad included)
            for (int i = tid; i < mc * per; i += MT_THREADS) {
                const int r = i / per, k8 = i - r * per;
                u32x4_t v = {0u, 0u, 0u, 0u};
                if (r < c && k8 < H / 8) {
                    const int p = ld_global(groups + (size_t)g * MT_GREC + 2 + r);
                    v = ld_global(reinterpret_cast<const u32x4_t *>(X + (size_t)(p / top_k) * H) + k8);
                }
                reinterpret_cast<u32x4_t *>(xl)[i] = v;
            }
            staged = g;
        }
        for (int i = tid; i < nr * MT_WAVES * 2 * 64; i += MT_THREADS) part[i] = 0.f;
        __syncthreads();
        const bool act = m < c;
        const uint16_t *arow = xl + (act ? m : 0) * XS + 32 * kg;
#pragma unroll 1
        for (;;) {
            if (t >= T) break;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                Fp4Batch &Cur = half ? B : A;
                Fp4Batch &Nxt = half ? A : B;
                const MtCursor cn = mt_advance(ca, nbu);
                const bool nvalid = t + MT_WAVES < T;
                const __amdgpu_buffer_rsrc_t rs =
                    mt_rsrc(cn.b < nb ? pg : pu, e, nrbF, rb0 + cn.i, PH, nvalid);
                const int tbn = (cn.b % nb) * MS_TPB, tbc = (ca.b % nb) * MS_TPB;
#pragma unroll
                for (int q = 0; q < MS_TPB; ++q) {
                    __builtin_amdgcn_sched_barrier(0);
                    fp4_tile_load(Nxt, q, rs, tbn + q, PH, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    mt_tile_x(Cur.c0[q], Cur.c1[q], Cur.e0[q], Cur.e1[q], arow, act, tbc + q, D0,
                              D1);
                }
                // flush at the wave's last batch of this unit's gate or up rows
                const bool gate = ca.b < nb;
                if (!nvalid || cn.i != ca.i || (gate && cn.b >= nb)) {
                    mt_flush(part + ((ca.i * MT_WAVES + wave) * 2 + (gate ? 0 : 1)) * 64, D0, D1,
                             lane);
                    D0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    D1 = D0;
                }
                t += MT_WAVES;
                ca = cn;
                if (t >= T) break;
            }
        }
        __syncthreads();
        for (int r = tid; r < nr * 64; r += MT_THREADS) {
            const int i = r >> 6, mm = (r >> 4) & 3, row = r & 15;
            if (mm >= c) continue;
            float gs = 0.f, us = 0.f;
#pragma unroll
            for (int w = 0; w < MT_WAVES; ++w) {
                gs += part[((i * MT_WAVES + w) * 2 + 0) * 64 + 16 * mm + row];
                us += part[((i * MT_WAVES + w) * 2 + 1) * 64 + 16 * mm + row];
            }
            const int p = ld_global(groups + (size_t)g * MT_GREC + 2 + mm);
            h_ws[(size_t)p * F + (rb0 + i) * RB + row] = gs / (1.f + expf(-gs)) * us;
        }
        ub += nr;
    }
}

// ------------------------------------------------------------ B: down
// Units u = g * nrbH + rb, nb batches each.  h of the group's pairs is
// staged as bf16 hi rows [0, mc) and lo rows [mc, 2 mc).
__global__ void __launch_bounds__(MT_THREADS, 2)
moe_t_down_kernel(const uint8_t *__restrict__ pd, const float *__restrict__ h_ws, int H, int F,
                  int PF, int nrbH, int mc, const int32_t *__restrict__ groups,
                  const unsigned *__restrict__ hdr, float *__restrict__ part_ws) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int nb = (PF + MS_TPB - 1) / MS_TPB;
    const int FS = nb * MS_TPB * 256 + 8;  // row stride (bf16), 16-byte pad
    uint16_t *hl = reinterpret_cast<uint16_t *>(smem);                         // [2][mc][FS]
    float *part = reinterpret_cast<float *>(smem + (size_t)2 * mc * FS * 2);  // [RMAX][W][64]
    const int tid = threadIdx.x, lane = tid & 63, kg = lane >> 4, m = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ng = __builtin_amdgcn_readfirstlane(ld_global(hdr + 1));
    const int64_t units = (int64_t)ng * nrbH, G = gridDim.x, j = blockIdx.x;
    const int u0 = (int)(j * units / G), u1 = (int)((j + 1) * units / G);
    int staged = -1;
#pragma unroll 1
    for (int ub = u0; ub < u1;) {
        const int g = ub / nrbH, rb0 = ub - g * nrbH;
        const int nr = min(min(u1 - ub, nrbH - rb0), MT_RMAX);
        const int2 gr = mt_group(groups, g);
        const int e = gr.x, c = gr.y;
        const int T = nr * nb;
        int t = wave;
        MtCursor ca = {t / nb, t % nb};
        Fp4Batch A, B;
        f32x4_t D0 = {0.f, 0.f, 0.f, 0.f}, D1 = D0;
        {
            const __amdgpu_buffer_rsrc_t rs = mt_rsrc(pd, e, nrbH, rb0 + ca.i, PF, t < T);
#pragma unroll
            for (int q = 0; q < MS_TPB; ++q) fp4_tile_load(A, q, rs, ca.b * MS_TPB + q, PF, lane);
        }
        __syncthreads();  // the previous block is done with h and part
        if (g != staged) {
            const int per = FS / 4;  // 4-element chunks per staged row (the pad included)
            for (int i = tid; i < mc * per; i += MT_THREADS) {
                const int r = i / per, k4 = i - r * per;
                f32x4_t v = {0.f, 0.f, 0.f, 0.f};
                if (r < c && k4 < F / 4) {
                    const int p = ld_global(groups + (size_t)g * MT_GREC + 2 + r);
                    v = ld_global(reinterpret_cast<const f32x4_t *>(h_ws + (size_t)p * F) + k4);
                }
                const float f[4] = {v[0], v[1], v[2], v[3]};
                uint16_t hi[4], lo[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    hi[q] = f32_to_bf16(f[q]);
                    lo[q] = f32_to_bf16(f[q] - __builtin_bit_cast(float, (unsigned)hi[q] << 16));
                }
                uint2 vh, vl;
                vh.x = hi[0] | ((unsigned)hi[1] << 16);
                vh.y = hi[2] | ((unsigned)hi[3] << 16);
                vl.x = lo[0] | ((unsigned)lo[1] << 16);
                vl.y = lo[2] | ((unsigned)lo[3] << 16);
                reinterpret_cast<uint2 *>(hl + (size_t)r * FS)[k4] = vh;
                reinterpret_cast<uint2 *>(hl + (size_t)(mc + r) * FS)[k4] = vl;
            }
            staged = g;
        }
        for (int i = tid; i < nr * MT_WAVES * 64; i += MT_THREADS) part[i] = 0.f;
        __syncthreads();
        const bool act = m < c;
        const uint16_t *ahi = hl + (act ? m : 0) * FS + 32 * kg;
        const uint16_t *alo = ahi + (size_t)mc * FS;
#pragma unroll 1
        for (;;) {
            if (t >= T) break;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                Fp4Batch &Cur = half ? B : A;
                Fp4Batch &Nxt = half ? A : B;
                const MtCursor cn = mt_advance(ca, nb);
                const bool nvalid = t + MT_WAVES < T;
                const __amdgpu_buffer_rsrc_t rs = mt_rsrc(pd, e, nrbH, rb0 + cn.i, PF, nvalid);
#pragma unroll
                for (int q = 0; q < MS_TPB; ++q) {
                    __builtin_amdgcn_sched_barrier(0);
                    fp4_tile_load(Nxt, q, rs, cn.b * MS_TPB + q, PF, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    mt_tile_h(Cur.c0[q], Cur.c1[q], Cur.e0[q], Cur.e1[q], ahi, alo, act,
                              ca.b * MS_TPB + q, D0, D1);
                }
                if (!nvalid || cn.i != ca.i) {
                    mt_flush(part + (ca.i * MT_WAVES + wave) * 64, D0, D1, lane);
                    D0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    D1 = D0;
                }
                t += MT_WAVES;
                ca = cn;
                if (t >= T) break;
            }
        }
        __syncthreads();
        for (int r = tid; r < nr * 64; r += MT_THREADS) {
            const int i = r >> 6, mm = (r >> 4) & 3, row = r & 15;
            if (mm >= c) continue;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < MT_WAVES; ++w) v += part[(i * MT_WAVES + w) * 64 + 16 * mm + row];
            const int p = ld_global(groups + (size_t)g * MT_GREC + 2 + mm);
            part_ws[(size_t)p * H + (rb0 + i) * RB + row] = v;
        }
        ub += nr;
    }
}

// Activation rows per group: as many (up to 4) as keep the staged x and the
// staged h of a workgroup within 64 KB each, so two workgroups fit on a CU.
int moe_skinny_group_rows(int64_t H, int64_t F) {
    const int64_t hpad = ceil_div(ceil_div(H, FP4_TILE_K), MS_TPB) * MS_TPB * 256 + 8;
    const int64_t fpad = ceil_div(ceil_div(F, FP4_TILE_K), MS_TPB) * MS_TPB * 256 + 8;
    int mc = MOE_GROUP_ROWS_MAX;
    while (mc > 1 && (mc * hpad * 2 > 65536 || 2 * mc * fpad * 2 > 65536)) --mc;
    return mc;
}

hipError_t launch_moe_skinny(const uint8_t *pg, const uint8_t *pu, const uint8_t *pd, int64_t E,
                             int64_t H, int64_t F, int T, const uint16_t *X, int top_k,
                             const int32_t *ids, const float *w, uint8_t *workspace, void *Y,
                             bool out_f32, int cus, hipStream_t s) {
    const int P = T * top_k;
    float *h_ws = reinterpret_cast<float *>(workspace);
    float *part = h_ws + (size_t)P * F;
    unsigned *hdr = reinterpret_cast<unsigned *>(part + (size_t)P * H);
    int32_t *groups = reinterpret_cast<int32_t *>(hdr + 4);
    const int mc = moe_skinny_group_rows(H, F);
    // always launched: it also rewrites the status word
    hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(MT_ROUTE_THREADS), 0, s, ids, P, (int)E,
                       mc, groups, hdr);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (P > 0) {
        const int PH = (int)ceil_div(H, FP4_TILE_K), nrbF = (int)(F / RB);
        const int nbA = (int)ceil_div(PH, MS_TPB);
        const int64_t unitsA = (int64_t)P * nrbF;
        const int gridA = (int)(unitsA < (int64_t)cus * 2 ? unitsA : (int64_t)cus * 2);
        const size_t ldsA = (size_t)mc * (nbA * MS_TPB * 256 + 8) * 2 +
                            (size_t)MT_RMAX * MT_WAVES * 2 * 64 * 4;
        hipLaunchKernelGGL(moe_t_gate_up_kernel, dim3(gridA), dim3(MT_THREADS), ldsA, s, pg, pu, X,
                           top_k, (int)H, (int)F, PH, nrbF, mc, groups, hdr, h_ws);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
        const int PF = (int)ceil_div(F, FP4_TILE_K), nrbH = (int)(H / RB);
        const int nbB = (int)ceil_div(PF, MS_TPB);
        const int64_t unitsB = (int64_t)P * nrbH;
        const int gridB = (int)(unitsB < (int64_t)cus * 2 ? unitsB : (int64_t)cus * 2);
        const size_t ldsB = (size_t)2 * mc * (nbB * MS_TPB * 256 + 8) * 2 +
                            (size_t)MT_RMAX * MT_WAVES * 64 * 4;
        hipLaunchKernelGGL(moe_t_down_kernel, dim3(gridB), dim3(MT_THREADS), ldsB, s, pd, h_ws,
                           (int)H, (int)F, PF, nrbH, mc, groups, hdr, part);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return launch_moe_combine(part, ids, w, E, H, top_k, T, Y, out_f32, nullptr, s);
}

}  // namespace qg
