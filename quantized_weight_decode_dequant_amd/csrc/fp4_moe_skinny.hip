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
// Each unit is computed by one wave, its tiles in K order, and written from
// its registers, so results are deterministic.
#include "fp4_stream.h"

namespace qg {

constexpr int MT_WAVES = 4;
constexpr int MT_THREADS = MT_WAVES * 64;
constexpr int MT_GREC = 8;          // int32 per group record: e, c, p[4], 0, 0
constexpr int MT_ROUTE_THREADS = 1024;

// ------------------------------------------------------------ R: routing
// key = expert id of a valid pair, -1 for an invalid one (-2 pads the arrays
// to a multiple of 4).  rank = pairs of the same expert before it; a pair
// whose rank is a multiple of mc starts a group, and the group index of a
// pair is the number of group starts of smaller expert ids plus rank / mc.
// Each count scans all pairs; the scans of one pair are split over up to
// 1024 / P threads, whose partial counts are added with integer LDS atomics
// (exact and order-independent).
__global__ void __launch_bounds__(MT_ROUTE_THREADS)
moe_route_kernel(const int32_t *__restrict__ ids, int P, int E, int mc,
                 int32_t *__restrict__ groups, unsigned *__restrict__ hdr) {
    __shared__ __attribute__((aligned(16))) int key[MOE_PAIRS_MAX];
    __shared__ __attribute__((aligned(16))) int start[MOE_PAIRS_MAX];
    __shared__ int rank[MOE_PAIRS_MAX], count[MOE_PAIRS_MAX], before[MOE_PAIRS_MAX];
    __shared__ unsigned s_bad, s_ng;
    const int tid = threadIdx.x;
    const int P4 = (P + 3) / 4;
    if (tid == 0) {
        s_bad = 0;
        s_ng = 0;
    }
    for (int p = tid; p < 4 * P4; p += MT_ROUTE_THREADS) {
        int k = -2;
        if (p < P) {
            const int e = ids[p];
            k = (e >= 0 && e < E) ? e : -1;
        }
        key[p] = k;
        start[p] = -1;
        rank[p] = 0;
        count[p] = 0;
        before[p] = 0;
    }
    __syncthreads();
    const int4 *key4 = reinterpret_cast<const int4 *>(key);
    const int4 *start4 = reinterpret_cast<const int4 *>(start);
    // slices per pair; work item w = slice * P + p
    const int S = P > 0 ? max(1, min(MT_ROUTE_THREADS / P, P4)) : 1;
    for (int w = tid; w < S * P; w += MT_ROUTE_THREADS) {
        const int sl = w / P, p = w - sl * P;
        const int kp = key[p];
        if (kp < 0) {
            if (sl == 0) atomicOr(&s_bad, 1u);
            continue;
        }
        const int q0 = sl * P4 / S, q1 = (sl + 1) * P4 / S;
        int r = 0, n = 0;
#pragma unroll 8
        for (int q4 = q0; q4 < q1; ++q4) {
            const int4 k = key4[q4];
            const int q = 4 * q4;
            n += (k.x == kp) + (k.y == kp) + (k.z == kp) + (k.w == kp);
            r += (k.x == kp && q < p) + (k.y == kp && q + 1 < p) + (k.z == kp && q + 2 < p) +
                 (k.w == kp && q + 3 < p);
        }
        atomicAdd(&rank[p], r);
        atomicAdd(&count[p], n);
    }
    __syncthreads();
    for (int p = tid; p < P; p += MT_ROUTE_THREADS) {
        const int kp = key[p];
        if (kp >= 0 && rank[p] % mc == 0) start[p] = kp;
    }
    __syncthreads();
    for (int w = tid; w < S * P; w += MT_ROUTE_THREADS) {
        const int sl = w / P, p = w - sl * P;
        const int kp = key[p];
        if (kp < 0) continue;
        const int q0 = sl * P4 / S, q1 = (sl + 1) * P4 / S;
        int b = 0;  // group starts of smaller expert ids
#pragma unroll 8
        for (int q4 = q0; q4 < q1; ++q4) {
            const int4 sq = start4[q4];
            b += (sq.x >= 0 && sq.x < kp) + (sq.y >= 0 && sq.y < kp) + (sq.z >= 0 && sq.z < kp) +
                 (sq.w >= 0 && sq.w < kp);
        }
        atomicAdd(&before[p], b);
    }
    __syncthreads();
    for (int p = tid; p < P; p += MT_ROUTE_THREADS) {
        const int kp = key[p];
        if (kp < 0) continue;
        const int r = rank[p], gid = before[p] + r / mc, slot = r % mc;
        int32_t *g = groups + (size_t)gid * MT_GREC;
        st_global<int32_t>(g, 2 + slot, p);
        if (slot == 0) {
            const int c = min(mc, count[p] - r);
            st_global<int32_t>(g, 0, kp);
            st_global<int32_t>(g, 1, c);
            for (int i = 2 + c; i < MT_GREC; ++i) st_global<int32_t>(g, i, 0);
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

// The A operands of one half of a tile: 4 (or, for split rows, 4 hi then 4
// lo) 8-element pieces of the lane's activation row, all read inside one
// branch so that the reads go out together and are waited for once; lanes
// whose row is not one of the group's keep zeros and read nothing.
__device__ __forceinline__ void lds_half(const uint16_t *a, bool act, bf16x8_t (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = bf16x8_t{};
    if (act) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const bf16x8_t *>(a + 8 * i);
    }
}
__device__ __forceinline__ void lds_half2(const uint16_t *ahi, const uint16_t *alo, bool act,
                                          bf16x8_t (&vh)[4], bf16x8_t (&vl)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        vh[i] = bf16x8_t{};
        vl[i] = bf16x8_t{};
    }
    if (act) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            vh[i] = *reinterpret_cast<const bf16x8_t *>(ahi + 8 * i);
            vl[i] = *reinterpret_cast<const bf16x8_t *>(alo + 8 * i);
        }
    }
}

// One tile (index tp of the staged rows) against one bf16 activation row per
// lane: arow = row (lane & 15) + 32 (lane >> 4); act = the row is one of the
// group's.  Half 0 accumulates into D0, half 1 into D1.
__device__ __forceinline__ void mt_tile_x(u32x4_t c0, u32x4_t c1, unsigned e0, unsigned e1,
                                          const uint16_t *arow, bool act, int tp, f32x4_t &D0,
                                          f32x4_t &D1) {
    const float s0 = e8m0_as_f32(e0), s1 = e8m0_as_f32(e1);
    const uint16_t *a = arow + 256 * tp;
    bf16x8_t v[4];
    lds_half(a, act, v);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        D0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[i], fp4_word_bf16x8(c0[i], s0), D0, 0, 0, 0);
    lds_half(a + 128, act, v);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        D1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[i], fp4_word_bf16x8(c1[i], s1), D1, 0, 0, 0);
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
        bf16x8_t vh[4], vl[4];
        lds_half2(ahi + o + 128 * jh, alo + o + 128 * jh, act, vh, vl);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x8_t B = fp4_word_bf16x8(c[i], sc);
            D0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vh[i], B, D0, 0, 0, 0);
            D1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vl[i], B, D1, 0, 0, 0);
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

// The group's pair ids (wave-uniform; entries past c are 0).
struct MtPairs {
    int p[MOE_GROUP_ROWS_MAX];
};
// Entry r (0 <= r < MOE_GROUP_ROWS_MAX; r may differ between lanes), chosen
// by selects among the wave-uniform entries (taken through readfirstlane so
// that the choice stays in registers rather than becoming an indexed load
// from a private array).
static_assert(MOE_GROUP_ROWS_MAX == 4, "mt_pair selects among 4 entries");
__device__ __forceinline__ int mt_pair(const MtPairs &pp, int r) {
    const int p0 = __builtin_amdgcn_readfirstlane(pp.p[0]);
    const int p1 = __builtin_amdgcn_readfirstlane(pp.p[1]);
    const int p2 = __builtin_amdgcn_readfirstlane(pp.p[2]);
    const int p3 = __builtin_amdgcn_readfirstlane(pp.p[3]);
    return r == 3 ? p3 : r == 2 ? p2 : r == 1 ? p1 : p0;
}
constexpr int MT_SU = 8;  // staging chunks per thread in flight

// Cached 16-byte buffer load (activations that other workgroups read too);
// an offset at or past the resource's range reads zero.
__device__ __forceinline__ u32x4_t buf_ld_x4_cached(__amdgpu_buffer_rsrc_t r, unsigned voff) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}
__device__ __forceinline__ MtPairs mt_pairs(const int32_t *groups, int g) {
    MtPairs r;
#pragma unroll
    for (int j = 0; j < MOE_GROUP_ROWS_MAX; ++j)
        r.p[j] = __builtin_amdgcn_readfirstlane(ld_global(groups + (size_t)g * MT_GREC + 2 + j));
    return r;
}

constexpr int MT_WAVES_A = 8, MT_THREADS_A = 512;
// ------------------------------------------------------------ A: gate / up
// Units u = g * nrbF + rb.  A workgroup's range of units is cut into blocks
// at group boundaries (x is restaged when the group changes); within a block
// wave w streams units w, w + 4, ..., each as nb batches of its gate rows
// then nb of its up rows, double-buffered across unit boundaries, and writes
// h = silu(g) u of the unit's rows for the group's pairs from registers.
__global__ void __launch_bounds__(MT_THREADS_A, 2)
moe_t_gate_up_kernel(const uint8_t *__restrict__ pg, const uint8_t *__restrict__ pu,
                     const uint16_t *__restrict__ X, int T_x, int top_k, int H, int F, int PH,
                     int nrbF, int mc, const int32_t *__restrict__ groups,
                     const unsigned *__restrict__ hdr, float *__restrict__ h_ws) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int nb = (PH + MS_TPB - 1) / MS_TPB, nbu = 2 * nb;
    const int XS = nb * MS_TPB * 256 + 8;  // row stride (bf16), 16-byte pad
    uint16_t *xl = reinterpret_cast<uint16_t *>(smem);  // [mc][XS]
    const int tid = threadIdx.x, lane = tid & 63, kg = lane >> 4, m = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ng = __builtin_amdgcn_readfirstlane(ld_global(hdr + 1));
    const int64_t units = (int64_t)ng * nrbF, G = gridDim.x, j = blockIdx.x;
    const int u0 = (int)(j * units / G), u1 = (int)((j + 1) * units / G);
    int staged = -1;
#pragma unroll 1
    for (int ub = u0; ub < u1;) {
        const int g = ub / nrbF, rb0 = ub - g * nrbF;
        const int nr = min(u1 - ub, nrbF - rb0);
        const int2 gr = mt_group(groups, g);
        const int e = gr.x, c = gr.y;
        const MtPairs pp = mt_pairs(groups, g);
        const int nu = nr > wave ? (nr - wave + MT_WAVES_A - 1) / MT_WAVES_A : 0;
        const int T = nu * nbu;  // this wave's batches in the block
        int ci = wave, cb = 0;   // current unit (block-relative) and batch
        Fp4Batch A, B;
        f32x4_t D0 = {0.f, 0.f, 0.f, 0.f}, D1 = D0, Gs = D0;
        {
            // the first batch loads while x is staged
            const __amdgpu_buffer_rsrc_t rs = mt_rsrc(pg, e, nrbF, rb0 + ci, PH, T > 0);
#pragma unroll
            for (int q = 0; q < MS_TPB; ++q) fp4_tile_load(A, q, rs, q, PH, lane);
        }
        __syncthreads();  // the previous block is done with x
        if (g != staged) {
            // 16-byte chunks per staged row (the pad included); each thread
            // issues the loads of MT_SU chunks before it writes any of them
            // (buffer loads: a chunk past the row or the group reads zero)
            const int per = XS / 8, n = mc * per;
            const unsigned xbytes = (unsigned)T_x * (unsigned)H * 2u;
            const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, xbytes);
            for (int i0 = tid; i0 < n; i0 += MT_SU * MT_THREADS_A) {
                u32x4_t v[MT_SU];
#pragma unroll
                for (int q = 0; q < MT_SU; ++q) {
                    const int i = i0 + q * MT_THREADS_A, r = i / per, k8 = i - r * per;
                    const bool ok = r < c && k8 < H / 8;
                    const unsigned off =
                        ok ? 2u * ((unsigned)(mt_pair(pp, r) / top_k) * (unsigned)H + 8u * k8)
                           : xbytes;
                    v[q] = buf_ld_x4_cached(rx, off);
                }
#pragma unroll
                for (int q = 0; q < MT_SU; ++q) {
                    const int i = i0 + q * MT_THREADS_A;
                    if (i < n) reinterpret_cast<u32x4_t *>(xl)[i] = v[q];
                }
            }
            staged = g;
        }
        __syncthreads();
        const bool act = m < c;
        const uint16_t *arow = xl + (act ? m : 0) * XS + 32 * kg;
#pragma unroll 1
        for (int t = 0; t < T;) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                Fp4Batch &Cur = half ? B : A;
                Fp4Batch &Nxt = half ? A : B;
                int ni = ci, nbx = cb + 1;
                if (nbx == nbu) {
                    nbx = 0;
                    ni += MT_WAVES_A;
                }
                const bool nvalid = t + 1 < T;
                const __amdgpu_buffer_rsrc_t rs =
                    mt_rsrc(nbx < nb ? pg : pu, e, nrbF, rb0 + ni, PH, nvalid);
                const int tbn = (nbx < nb ? nbx : nbx - nb) * MS_TPB;
                const int tbc = (cb < nb ? cb : cb - nb) * MS_TPB;
#pragma unroll
                for (int q = 0; q < MS_TPB; ++q) {
                    __builtin_amdgcn_sched_barrier(0);
                    fp4_tile_load(Nxt, q, rs, tbn + q, PH, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    mt_tile_x(Cur.c0[q], Cur.c1[q], Cur.e0[q], Cur.e1[q], arow, act, tbc + q, D0,
                              D1);
                }
                if (cb == nb - 1) {  // the unit's gate rows are done
                    Gs = D0 + D1;
                    D0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    D1 = D0;
                } else if (cb == nbu - 1) {  // up rows done: h of the unit's rows
                    const f32x4_t Us = D0 + D1;
                    if (lane < 16) {
                        const size_t row = (size_t)(rb0 + ci) * RB + lane;
#pragma unroll
                        for (int r = 0; r < MOE_GROUP_ROWS_MAX; ++r)
                            if (r < c)
                                st_global<float>(h_ws, (size_t)pp.p[r] * F + row,
                                                 Gs[r] / (1.f + expf(-Gs[r])) * Us[r]);
                    }
                    D0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    D1 = D0;
                }
                ci = ni;
                cb = nbx;
                ++t;
                if (t >= T) break;
            }
        }
        ub += nr;
    }
}

// ------------------------------------------------------------ B: down
// Units u = g * nrbH + rb, nb batches each, streamed per wave as in A; h of
// the group's pairs is staged as bf16 hi rows [0, mc) and lo rows [mc, 2 mc).
__global__ void __launch_bounds__(MT_THREADS, 3)
moe_t_down_kernel(const uint8_t *__restrict__ pd, const float *__restrict__ h_ws, int P, int H,
                  int F, int PF, int nrbH, int mc, const int32_t *__restrict__ groups,
                  const unsigned *__restrict__ hdr, float *__restrict__ part_ws) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int nb = (PF + MS_TPB - 1) / MS_TPB;
    const int FS = nb * MS_TPB * 256 + 8;  // row stride (bf16), 16-byte pad
    uint16_t *hl = reinterpret_cast<uint16_t *>(smem);  // [2][mc][FS]
    const int tid = threadIdx.x, lane = tid & 63, kg = lane >> 4, m = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ng = __builtin_amdgcn_readfirstlane(ld_global(hdr + 1));
    const int64_t units = (int64_t)ng * nrbH, G = gridDim.x, j = blockIdx.x;
    const int u0 = (int)(j * units / G), u1 = (int)((j + 1) * units / G);
    int staged = -1;
#pragma unroll 1
    for (int ub = u0; ub < u1;) {
        const int g = ub / nrbH, rb0 = ub - g * nrbH;
        const int nr = min(u1 - ub, nrbH - rb0);
        const int2 gr = mt_group(groups, g);
        const int e = gr.x, c = gr.y;
        const MtPairs pp = mt_pairs(groups, g);
        const int nu = nr > wave ? (nr - wave + MT_WAVES - 1) / MT_WAVES : 0;
        const int T = nu * nb;
        int ci = wave, cb = 0;
        Fp4Batch A, B;
        f32x4_t D0 = {0.f, 0.f, 0.f, 0.f}, D1 = D0;
        {
            const __amdgpu_buffer_rsrc_t rs = mt_rsrc(pd, e, nrbH, rb0 + ci, PF, T > 0);
#pragma unroll
            for (int q = 0; q < MS_TPB; ++q) fp4_tile_load(A, q, rs, q, PF, lane);
        }
        __syncthreads();  // the previous block is done with h
        if (g != staged) {
            // 4-element chunks per staged row (the pad included); each thread
            // issues the loads of MT_SU chunks before it converts any of them
            // (buffer loads: a chunk past the row or the group reads zero)
            const int per = FS / 4, n = mc * per;
            const unsigned hbytes = (unsigned)P * (unsigned)F * 4u;
            const __amdgpu_buffer_rsrc_t rh = make_rsrc(h_ws, hbytes);
            for (int i0 = tid; i0 < n; i0 += MT_SU * MT_THREADS) {
                f32x4_t vv[MT_SU];
#pragma unroll
                for (int q = 0; q < MT_SU; ++q) {
                    const int i = i0 + q * MT_THREADS, r = i / per, k4 = i - r * per;
                    const bool ok = r < c && k4 < F / 4;
                    const unsigned off =
                        ok ? 4u * ((unsigned)mt_pair(pp, r) * (unsigned)F + 4u * k4) : hbytes;
                    vv[q] = __builtin_bit_cast(f32x4_t, buf_ld_x4_cached(rh, off));
                }
#pragma unroll
                for (int q = 0; q < MT_SU; ++q) {
                    const int i = i0 + q * MT_THREADS, r = i / per, k4 = i - r * per;
                    if (i >= n) continue;
                    uint16_t hi[4], lo[4];
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4) {
                        const float f = vv[q][e4];
                        hi[e4] = f32_to_bf16(f);
                        lo[e4] = f32_to_bf16(f - __builtin_bit_cast(float, (unsigned)hi[e4] << 16));
                    }
                    uint2 vh, vl;
                    vh.x = hi[0] | ((unsigned)hi[1] << 16);
                    vh.y = hi[2] | ((unsigned)hi[3] << 16);
                    vl.x = lo[0] | ((unsigned)lo[1] << 16);
                    vl.y = lo[2] | ((unsigned)lo[3] << 16);
                    reinterpret_cast<uint2 *>(hl + (size_t)r * FS)[k4] = vh;
                    reinterpret_cast<uint2 *>(hl + (size_t)(mc + r) * FS)[k4] = vl;
                }
            }
            staged = g;
        }
        __syncthreads();
        const bool act = m < c;
        const uint16_t *ahi = hl + (act ? m : 0) * FS + 32 * kg;
        const uint16_t *alo = ahi + (size_t)mc * FS;
#pragma unroll 1
        for (int t = 0; t < T;) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                Fp4Batch &Cur = half ? B : A;
                Fp4Batch &Nxt = half ? A : B;
                int ni = ci, nbx = cb + 1;
                if (nbx == nb) {
                    nbx = 0;
                    ni += MT_WAVES;
                }
                const bool nvalid = t + 1 < T;
                const __amdgpu_buffer_rsrc_t rs = mt_rsrc(pd, e, nrbH, rb0 + ni, PF, nvalid);
#pragma unroll
                for (int q = 0; q < MS_TPB; ++q) {
                    __builtin_amdgcn_sched_barrier(0);
                    fp4_tile_load(Nxt, q, rs, nbx * MS_TPB + q, PF, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    mt_tile_h(Cur.c0[q], Cur.c1[q], Cur.e0[q], Cur.e1[q], ahi, alo, act,
                              cb * MS_TPB + q, D0, D1);
                }
                if (cb == nb - 1) {  // the unit is done
                    const f32x4_t Ys = D0 + D1;
                    if (lane < 16) {
                        const size_t row = (size_t)(rb0 + ci) * RB + lane;
#pragma unroll
                        for (int r = 0; r < MOE_GROUP_ROWS_MAX; ++r)
                            if (r < c) st_global<float>(part_ws, (size_t)pp.p[r] * H + row, Ys[r]);
                    }
                    D0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    D1 = D0;
                }
                ci = ni;
                cb = nbx;
                ++t;
                if (t >= T) break;
            }
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
        const size_t ldsA = (size_t)mc * (nbA * MS_TPB * 256 + 8) * 2;
        hipLaunchKernelGGL(moe_t_gate_up_kernel, dim3(gridA), dim3(MT_THREADS_A), ldsA, s, pg, pu, X,
                           T, top_k, (int)H, (int)F, PH, nrbF, mc, groups, hdr, h_ws);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
        const int PF = (int)ceil_div(F, FP4_TILE_K), nrbH = (int)(H / RB);
        const int nbB = (int)ceil_div(PF, MS_TPB);
        const int64_t unitsB = (int64_t)P * nrbH;
        const int gridB = (int)(unitsB < (int64_t)cus * 3 ? unitsB : (int64_t)cus * 3);
        const size_t ldsB = (size_t)2 * mc * (nbB * MS_TPB * 256 + 8) * 2;
        hipLaunchKernelGGL(moe_t_down_kernel, dim3(gridB), dim3(MT_THREADS), ldsB, s, pd, h_ws, P,
                           (int)H, (int)F, PF, nrbH, mc, groups, hdr, part);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return launch_moe_combine(part, ids, w, E, H, top_k, T, Y, out_f32, nullptr, s);
}

}  // namespace qg
