// The affine weight family of "MLX Runner: An Inference Engine You Can Read"
// (section "Architecture: one command buffer per token": codes with a scale
// and a bias per group, w = scale * code + bias; the audit section lists the
// widths): unsigned codes of 2, 3, 4, 5, 6 or 8 bits, groups of 32, 64 or 128
// consecutive k, scale and bias in fp16 or bf16.  Packing and the decode GEMV
// y = W x for one bf16 activation row.
//
// Codes are stored as bit-planes of width 1, 2 or 4 (layout in
// qg_internal.h) with the two codes of a pair in the two 16-bit halves of a
// word, so one shift and one and-or per plane give a pair of small integers,
// and or-ing in 0x4300 makes each half the exact bf16 value 128 + q (q < 128).
// A lane's 32 codes are four runs of 8 consecutive k, one per 32-k block of
// the tile.  The GEMV accumulates (128 + q) x over a run with
// v_dot2_f32_bf16, and per group adds scale * (acc - 128 sum x) + bias * sum
// x, with sum x over the lane's k of that group staged once.  2- and 3-bit
// codes, whose unpacking costs the most VALU work per byte, take each run as
// the B operand of one v_mfma_f32_16x16x32_bf16 step against x (the same x
// in all 16 rows of A) instead: the matrix unit does the multiply-adds and
// the sum over the k-slices, the VALU only the unpack.  8-bit codes do
// not fit 128 + q in bf16: their two nibble planes run as two dot chains,
// D = D_lo + 16 D_hi.  The skinny product (M <= 32 rows) takes each run as
// the B operand of one v_mfma_f32_16x16x32_bf16 step (the 64 lanes' runs i
// make up the 32-k block i) against X staged in LDS, and applies the group's
// scale and bias to the step sums.
//
// Work split as in the other streaming GEMVs: contiguous ranges of rowblocks
// per workgroup, batches of 4 tiles round-robin over 4 waves, double-buffered,
// wave sums folded in LDS and added in wave order per block of 32 rowblocks.
#include "affine_tile.h"

namespace qg {

struct PlaneSpec {
    int np, w[2], o[2];
};
__host__ __device__ inline PlaneSpec plane_spec(int bits) {
    switch (bits) {
    case 2: return {1, {2, 0}, {0, 0}};
    case 3: return {2, {2, 1}, {0, 2}};
    case 4: return {1, {4, 0}, {0, 0}};
    case 5: return {2, {4, 1}, {0, 4}};
    case 6: return {2, {4, 2}, {0, 4}};
    default: return {2, {4, 4}, {0, 4}};  // 8
    }
}

size_t affine_packed_bytes(int bits, int group, int64_t N, int64_t K) {
    return (size_t)ceil_div(N, RB) * (size_t)ceil_div(K, AFF_TILE_K) *
           affine_tile_bytes(bits, group);
}

// ------------------------------------------------------------ packing
// One thread per (tile, lane) writes the lane's plane words; one thread per
// (tile, row, group) writes a (scale, bias) word.
__global__ void __launch_bounds__(256)
pack_affine_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                   const uint16_t *__restrict__ biases, int bits, int group, int64_t N, int64_t K,
                   int64_t P, int64_t nthreads, uint8_t *__restrict__ out) {
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= nthreads) return;
    const int gpt = AFF_TILE_K / group;  // groups per tile
    const int per_tile = 64 + 16 * gpt;
    const int64_t tile = id / per_tile;
    const int sub = (int)(id - tile * per_tile);
    const int64_t rb = tile / P, p = tile - rb * P;
    const size_t tb = affine_tile_bytes(bits, group);
    uint8_t *base = out + (size_t)tile * tb;
    const int64_t G = K / group;
    if (sub < 64) {
        const int l = sub;
        const int64_t n = rb * RB + (l & 15);
        // code 8i + t of the lane is k = 32i + 8(l >> 4) + t of the tile
        const int64_t kt = p * AFF_TILE_K;
        uint8_t c[32];
        for (int i = 0; i < 32; ++i) {
            const int64_t k = kt + 32 * (i >> 3) + 8 * (l >> 4) + (i & 7);
            c[i] = (n < N && k < K) ? codes[n * K + k] : 0;
        }
        const PlaneSpec ps = plane_spec(bits);
        size_t off = 0;
        for (int q = 0; q < ps.np; ++q) {
            const int w = ps.w[q], o = ps.o[q], per_word = 16 / w;
            const unsigned m = (1u << w) - 1u;
            for (int wi = 0; wi < w; ++wi) {
                unsigned word = 0;
                for (int s = 0; s < per_word; ++s) {
                    const int j = wi * per_word + s;
                    // 3-bit codes: bit 2 of pair j at ag3_pos(j) (affine_tile.h)
                    const int b = (bits == 3 && q == 1) ? ag3_pos(j) : w * s;
                    word |= (((unsigned)c[2 * j] >> o) & m) << b;
                    word |= (((unsigned)c[2 * j + 1] >> o) & m) << (16 + b);
                }
                reinterpret_cast<uint32_t *>(base + off + (size_t)4 * w * l)[wi] = word;
            }
            off += (size_t)256 * w;
        }
    } else {
        const int e = sub - 64, r = e / gpt, t = e - r * gpt;
        const int64_t n = rb * RB + r;
        const int64_t gi = p * gpt + t;
        unsigned word = 0;
        if (n < N && gi < G)
            word = (unsigned)scales[n * G + gi] | ((unsigned)biases[n * G + gi] << 16);
        reinterpret_cast<uint32_t *>(base + (size_t)256 * bits)[e] = word;
    }
}

hipError_t launch_pack_affine(const uint8_t *codes, const uint16_t *scales,
                              const uint16_t *biases, int bits, int group, int64_t N, int64_t K,
                              uint8_t *packed, hipStream_t s) {
    const int64_t P = ceil_div(K, AFF_TILE_K);
    const int64_t nthreads = ceil_div(N, RB) * P * (64 + 16 * (AFF_TILE_K / group));
    hipLaunchKernelGGL(pack_affine_kernel, dim3((unsigned)ceil_div(nthreads, 256)), dim3(256), 0,
                       s, codes, scales, biases, bits, group, N, K, P, nthreads, packed);
    return hipGetLastError();
}

// ------------------------------------------------------------ GEMV
constexpr int AG_WAVES = 4;
constexpr int AG_THREADS = AG_WAVES * 64;
constexpr int AG_TPB = 4;    // tiles per batch
constexpr int AG_RMAX = 32;  // rowblocks per output block

template <int BITS, int GPT>
struct AgBatch {
    AgTile<BITS, GPT> t[AG_TPB];
};

// 2- and 3-bit codes with fewer shifts.  The bf16 exponent decides where a
// code's bits sit in the mantissa: with the exponent of 128 a code in bits
// 0-2 reads as 128 + q, with that of 32 a code in bits 2-4 as 32 + q, with
// that of 8 a code in bits 4-6 as 8 + q.  So one plane-0 word (2-bit fields)
// gives the pairs at its positions 0, 1, 2 by masking alone, its copy shifted
// by 6 those at 3, 4, 5 and its copy shifted by 12 those at 6, 7: two shifts
// per word instead of seven.  A 3-bit code's plane-1 bit is shifted to just
// above its plane-0 field and merged in.  The dot products then carry
// sum_k off(k) x_k, off = 128, 32 or 8 by position, which is staged per
// group beside the plain sums of x.
constexpr bool ag_inplace(int bits) { return bits <= 3; }

struct Ag2Consts {
    unsigned m[3], g[3], b[3];
};

template <int BITS>
__device__ __forceinline__ Ag2Consts ag2_consts() {
    Ag2Consts k{{ag_opaque(0x00030003u), ag_opaque(0x000C000Cu), ag_opaque(0x00300030u)},
                {ag_opaque(0x43004300u), ag_opaque(0x42004200u), ag_opaque(0x41004100u)},
                {0u, 0u, 0u}};
    if constexpr (BITS == 3) {
        k.b[0] = ag_opaque(0x00040004u);
        k.b[1] = ag_opaque(0x00100010u);
        k.b[2] = ag_opaque(0x00400040u);
    }
    return k;
}

// The offset of pair position s (0..7) of a plane-0 word.
__host__ __device__ constexpr float ag2_off(int s) {
    return s % 3 == 0 ? 128.f : s % 3 == 1 ? 32.f : 8.f;
}

// Pair j (0..15, compile-time once unrolled): off(j % 8) + q in both halves.
template <int BITS, int GPT>
__device__ __forceinline__ unsigned ag2_pair(const AgTile<BITS, GPT> &T, int j,
                                             const Ag2Consts &k) {
    const unsigned w = T.p0[j / 8];
    const int s = j % 8, r = s % 3;
    const unsigned u = s < 3 ? w : s < 6 ? w >> 6 : w >> 12;
    if constexpr (BITS == 3) {
        const unsigned w1 = T.p1[0];
        const int sh = ag3_pos(j) - (2 * r + 2);  // pair j's plane-1 bit goes to bit 2 r + 2
        return ((sh >= 0 ? w1 >> sh : w1 << -sh) & k.b[r]) | ag_and_or(u, k.m[r], k.g[r]);
    } else {
        return (u & k.m[r]) | k.g[r];
    }
}

// One tile (4-, 5-, 6- and 8-bit codes): xrun = the lane's x of run 0 (run
// i at xrun + 32 i, 8 bf16), xg = the sums of the lane's x over each of the
// tile's GPT groups.  One dot chain per group; returns y plus the lane's
// share of the tile.
template <int BITS, int GPT, bool BF16S>
__device__ __forceinline__ float ag_tile(const AgTile<BITS, GPT> &T, const uint16_t *xrun,
                                         const float *xg, float y, const AgConsts &k) {
    constexpr int CPG = 4 / GPT;  // runs per group
#pragma unroll
    for (int t = 0; t < GPT; ++t) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int c = 0; c < CPG; ++c) {
            const int i = t * CPG + c;
            const uint4 xv = *reinterpret_cast<const uint4 *>(xrun + 32 * i);
            const unsigned xp[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                a0 = dot2_bf16(ag_bf16_pair<BITS, GPT>(T, 4 * i + h, k), xp[h], a0);
                if constexpr (BITS == 8)
                    a1 = dot2_bf16(ag_pair_hi<BITS, GPT>(T, 4 * i + h, k), xp[h], a1);
            }
        }
        const float X = xg[t];
        float D = fmaf(-128.f, X, a0);
        if constexpr (BITS == 8) D = fmaf(16.f, fmaf(-128.f, X, a1), D);
        const unsigned sb = T.sb[t];
        y = fmaf(ag_scale(sb, BF16S), D, fmaf(ag_bias(sb, BF16S), X, y));
    }
    return y;
}

// 2- and 3-bit codes: the dot products of a 32-k run on the bf16 MFMA, x as
// the A operand (the same in all 16 rows), the lane's 8 codes as its B column:
// every lane gets its row's dot over all four k-slices, so no shuffle folds
// them.  xg, xw: the sums of x (plain and offset-weighted) over each of the
// tile's GPT groups.
template <int BITS, int GPT, bool BF16S>
__device__ __forceinline__ float ag_tile_mfma(const AgTile<BITS, GPT> &T, const uint16_t *xrun,
                                              const float *xg, const float *xw, float y,
                                              const Ag2Consts &k2) {
    constexpr int CPG = 4 / GPT;  // runs per group
#pragma unroll
    for (int t = 0; t < GPT; ++t) {
        f32x4_t C = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < CPG; ++c) {
            const int i = t * CPG + c;
            const bf16x8_t A = *reinterpret_cast<const bf16x8_t *>(xrun + 32 * i);
            const u32x4_t b = {ag2_pair<BITS, GPT>(T, 4 * i, k2), ag2_pair<BITS, GPT>(T, 4 * i + 1, k2),
                               ag2_pair<BITS, GPT>(T, 4 * i + 2, k2),
                               ag2_pair<BITS, GPT>(T, 4 * i + 3, k2)};
            C = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8_t, b), C, 0, 0,
                                                        0);
        }
        const unsigned sb = T.sb[t];
        y = fmaf(ag_scale(sb, BF16S), C[0] - xw[t], fmaf(ag_bias(sb, BF16S), xg[t], y));
    }
    return y;
}

__device__ __forceinline__ float ag_reduce_kslices(float a) {
    a += __shfl_xor(a, 16);
    a += __shfl_xor(a, 32);
    return a;
}

// LDS of a workgroup: the partial sums first, at a fixed offset, so that a
// work-list workgroup can stage the next product's x while other waves still
// read the previous product's sums; then x and its group sums.
constexpr size_t AG_LDS_PART = (size_t)AG_RMAX * AG_WAVES * 16 * 4;

template <int BITS, int GPT>
static size_t ag_lds_bytes(int64_t K) {
    const int64_t KS = ceil_div(ceil_div(K, AFF_TILE_K), AG_TPB) * AG_TPB * AFF_TILE_K;
    // x sums: per (tile, k-slice, group) for the dot chains; per (tile,
    // group), plain and offset-weighted, for the MFMA path
    const int64_t nsum = ag_inplace(BITS) ? 2 * (KS / AFF_TILE_K) * GPT : (KS / 32) * GPT;
    return AG_LDS_PART + (size_t)KS * 2 + (size_t)nsum * 4;
}

// Rowblocks [u0, u1) of one product.
template <int BITS, int GPT, bool BF16S>
__device__ __forceinline__ void ag_range(const WorkItem &it, int u0, int u1, unsigned char *smem,
                                         int tid, int lane, int wave) {
    const uint8_t *__restrict__ packed = it.packed;
    const uint16_t *__restrict__ x = reinterpret_cast<const uint16_t *>(it.x);
    const int N = it.N, K = it.K, P = it.P;
    const int kg = lane >> 4;
    const int nb = (P + AG_TPB - 1) / AG_TPB;
    const int KS = nb * AG_TPB * AFF_TILE_K;  // staged x length (zero past K)
    float *part = reinterpret_cast<float *>(smem);                               // [RMAX][WAVES][16]
    uint16_t *xl = reinterpret_cast<uint16_t *>(smem + AG_LDS_PART);             // [KS] bf16
    // x sums: [KS / 32 * GPT] per (tile, k-slice, group); 2- and 3-bit codes:
    // [KS / 128 * GPT] per (tile, group), then the offset-weighted ones xwl
    float *xsl = reinterpret_cast<float *>(smem + AG_LDS_PART + (size_t)KS * 2);
    float *xwl = xsl + KS / AFF_TILE_K * GPT;
    const unsigned tb = (unsigned)affine_tile_bytes(BITS, AFF_TILE_K / GPT);
    const size_t rb_bytes = (size_t)P * tb;
    const AgConsts kc = ag_consts<BITS>();
    Ag2Consts k2{};
    if constexpr (ag_inplace(BITS)) k2 = ag2_consts<BITS>();
    // stage x, then the sum of each lane-group's x over each group of each
    // tile (its runs in k order, each run's 8 values in a fixed tree):
    // xsl[(4 tp + kg) GPT + t]; for 2- and 3-bit codes also the offset-weighted sums
    // xwl, pair h of run i weighted by ag2_off(4 (i % 2) + h)
    for (int c = tid; c < KS / 8; c += AG_THREADS) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (8 * c < K) v = reinterpret_cast<const uint4 *>(x)[c];
        reinterpret_cast<uint4 *>(xl)[c] = v;
    }
    __syncthreads();
    if constexpr (ag_inplace(BITS)) {
        // sums over each group of each tile (all four k-slices)
        for (int e = tid; e < KS / AFF_TILE_K * GPT; e += AG_THREADS) {
            const int t = e % GPT, tp = e / GPT;
            float sum = 0.f, wsum = 0.f;
#pragma unroll
            for (int ckg = 0; ckg < 4; ++ckg) {
#pragma unroll
                for (int c = 0; c < 4 / GPT; ++c) {
                    const int i = t * (4 / GPT) + c;
                    const uint4 v =
                        *reinterpret_cast<const uint4 *>(xl + tp * AFF_TILE_K + 32 * i + 8 * ckg);
                    const float p0 = bf16_lo(v.x) + bf16_hi(v.x), p1 = bf16_lo(v.y) + bf16_hi(v.y);
                    const float p2 = bf16_lo(v.z) + bf16_hi(v.z), p3 = bf16_lo(v.w) + bf16_hi(v.w);
                    const int s0 = 4 * (i % 2);
                    sum += (p0 + p1) + (p2 + p3);
                    wsum += (ag2_off(s0) * p0 + ag2_off(s0 + 1) * p1) +
                            (ag2_off(s0 + 2) * p2 + ag2_off(s0 + 3) * p3);
                }
            }
            xsl[e] = sum;
            xwl[e] = wsum;
        }
    } else {
        for (int e = tid; e < KS / 32 * GPT; e += AG_THREADS) {
            const int t = e % GPT, tk = e / GPT, tp = tk >> 2, ckg = tk & 3;
            float sum = 0.f;
#pragma unroll
            for (int c = 0; c < 4 / GPT; ++c) {
                const int i = t * (4 / GPT) + c;
                const uint4 v =
                    *reinterpret_cast<const uint4 *>(xl + tp * AFF_TILE_K + 32 * i + 8 * ckg);
                const float p0 = bf16_lo(v.x) + bf16_hi(v.x), p1 = bf16_lo(v.y) + bf16_hi(v.y);
                const float p2 = bf16_lo(v.z) + bf16_hi(v.z), p3 = bf16_lo(v.w) + bf16_hi(v.w);
                sum += (p0 + p1) + (p2 + p3);
            }
            xsl[e] = sum;
        }
    }
#pragma unroll 1
    for (int ub = u0; ub < u1; ub += AG_RMAX) {
        const int nr = min(u1 - ub, AG_RMAX);
        const int T = nr * nb;
        // wave w takes the batches whose absolute index (rowblock * nb +
        // batch) is w mod AG_WAVES, so a rowblock's split over the waves, and
        // hence its rounding, does not depend on where the workgroup's range
        // starts: single and grouped launches agree bit for bit
        int t = (wave - (int)(((int64_t)ub * nb) % AG_WAVES) + AG_WAVES) % AG_WAVES;
        int ci = t / nb, cb = t % nb;
        AgBatch<BITS, GPT> A, B;
        float acc = 0.f;
        {
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc(uniform_ptr(packed + (size_t)(ub + ci) * rb_bytes),
                          t < T ? (unsigned)rb_bytes : 0u);
#pragma unroll
            for (int q = 0; q < AG_TPB; ++q)
                ag_tile_load<BITS, GPT>(A.t[q], rs, cb * AG_TPB + q, P, tb, lane);
        }
        __syncthreads();  // x staged; the previous block's partial sums are read
        for (int i = tid; i < nr * AG_WAVES * 16; i += AG_THREADS) part[i] = 0.f;
        __syncthreads();
#pragma unroll 1
        for (;;) {
            if (t >= T) break;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                AgBatch<BITS, GPT> &Cur = half ? B : A;
                AgBatch<BITS, GPT> &Nxt = half ? A : B;
                int ni = ci, nbx = cb + AG_WAVES;
                while (nbx >= nb) {  // uniform
                    nbx -= nb;
                    ++ni;
                }
                const bool nvalid = t + AG_WAVES < T;
                const __amdgpu_buffer_rsrc_t rs =
                    make_rsrc(uniform_ptr(packed + (size_t)(ub + (nvalid ? ni : ci)) * rb_bytes),
                              nvalid ? (unsigned)rb_bytes : 0u);
#pragma unroll
                for (int q = 0; q < AG_TPB; ++q) {
                    __builtin_amdgcn_sched_barrier(0);
                    ag_tile_load<BITS, GPT>(Nxt.t[q], rs, nbx * AG_TPB + q, P, tb, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    const int tp = cb * AG_TPB + q;
                    if constexpr (ag_inplace(BITS))
                        acc = ag_tile_mfma<BITS, GPT, BF16S>(Cur.t[q], xl + tp * AFF_TILE_K + 8 * kg,
                                                             xsl + tp * GPT, xwl + tp * GPT, acc, k2);
                    else
                        acc = ag_tile<BITS, GPT, BF16S>(Cur.t[q], xl + tp * AFF_TILE_K + 8 * kg,
                                                        xsl + (4 * tp + kg) * GPT, acc, kc);
                }
                if (!nvalid || ni != ci) {  // the wave's last batch of this rowblock
                    if constexpr (!ag_inplace(BITS)) acc = ag_reduce_kslices(acc);
                    if (lane < 16) part[(ci * AG_WAVES + wave) * 16 + lane] += acc;
                    acc = 0.f;
                }
                t += AG_WAVES;
                ci = ni;
                cb = nbx;
                if (t >= T) break;
            }
        }
        __syncthreads();
        for (int r = tid; r < nr * 16; r += AG_THREADS) {
            const int i = r >> 4, row = r & 15;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < AG_WAVES; ++w) v += part[(i * AG_WAVES + w) * 16 + row];
            const int n = (ub + i) * RB + row;
            if (n < N) {
                if (it.out_f32)
                    st_global<float>(it.y, n, v);
                else
                    st_global<uint16_t>(it.y, n, f32_to_bf16(v));
            }
        }
    }
}

// LIST = false: one product (`single`), a contiguous share of its rowblocks
// per workgroup; LIST = true: the work list, workgroup j taking the units
// [starts[j], starts[j+1]).  Separate instantiations, so profiles tell a
// grouped launch from single GEMVs.
template <bool LIST, int BITS, int GPT, bool BF16S>
__global__ void __launch_bounds__(AG_THREADS, 4)
affine_gemv_kernel(const WorkItem *__restrict__ items, const WorkStart *__restrict__ starts,
                   WorkItem single) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (!LIST) {
        const int64_t n = single.units, g = gridDim.x, j = blockIdx.x;
        const int u0 = (int)(j * n / g), u1 = (int)((j + 1) * n / g);
        if (u0 < u1) ag_range<BITS, GPT, BF16S>(single, u0, u1, smem, tid, lane, wave);
        return;
    }
    const WorkStart s = starts[blockIdx.x], e = starts[blockIdx.x + 1];
#pragma unroll 1
    for (int i = s.item; i < e.item || (i == e.item && e.unit > 0); ++i) {
        const WorkItem it = items[i];
        const int u0 = (i == s.item) ? s.unit : 0;
        const int u1 = (i == e.item) ? e.unit : it.units;
        if (u0 < u1) ag_range<BITS, GPT, BF16S>(it, u0, u1, smem, tid, lane, wave);
    }
}

template <bool LIST, int BITS, int GPT>
static hipError_t launch_ag(const WorkItem *items, const WorkStart *starts, const WorkItem &it,
                            int grid, int64_t kmax, bool bf16, hipStream_t s) {
    const size_t lds = ag_lds_bytes<BITS, GPT>(kmax);
    if (bf16)
        hipLaunchKernelGGL((affine_gemv_kernel<LIST, BITS, GPT, true>), dim3(grid),
                           dim3(AG_THREADS), lds, s, items, starts, it);
    else
        hipLaunchKernelGGL((affine_gemv_kernel<LIST, BITS, GPT, false>), dim3(grid),
                           dim3(AG_THREADS), lds, s, items, starts, it);
    return hipGetLastError();
}

template <bool LIST, int BITS>
static hipError_t launch_ag_bits(const WorkItem *items, const WorkStart *starts,
                                 const WorkItem &it, int grid, int64_t kmax, int group, bool bf16,
                                 hipStream_t s) {
    switch (group) {
    case 32: return launch_ag<LIST, BITS, 4>(items, starts, it, grid, kmax, bf16, s);
    case 64: return launch_ag<LIST, BITS, 2>(items, starts, it, grid, kmax, bf16, s);
    default: return launch_ag<LIST, BITS, 1>(items, starts, it, grid, kmax, bf16, s);
    }
}

template <bool LIST>
static hipError_t launch_ag_fmt(const WorkItem *items, const WorkStart *starts,
                                const WorkItem &it, int grid, int64_t kmax, int bits, int group,
                                bool bf16, hipStream_t s) {
    switch (bits) {
    case 2: return launch_ag_bits<LIST, 2>(items, starts, it, grid, kmax, group, bf16, s);
    case 3: return launch_ag_bits<LIST, 3>(items, starts, it, grid, kmax, group, bf16, s);
    case 4: return launch_ag_bits<LIST, 4>(items, starts, it, grid, kmax, group, bf16, s);
    case 5: return launch_ag_bits<LIST, 5>(items, starts, it, grid, kmax, group, bf16, s);
    case 6: return launch_ag_bits<LIST, 6>(items, starts, it, grid, kmax, group, bf16, s);
    case 8: return launch_ag_bits<LIST, 8>(items, starts, it, grid, kmax, group, bf16, s);
    default: return hipErrorInvalidValue;
    }
}

int affine_gemv_wgs_per_cu() { return 4; }

hipError_t launch_affine_gemv(const uint8_t *packed, const uint16_t *x, void *y, int bits,
                              int group, bool bf16_scales, int64_t N, int64_t K, bool out_f32,
                              int cus, hipStream_t s) {
    WorkItem it{};
    it.packed = packed;
    it.x = x;
    it.y = y;
    it.N = (int32_t)N;
    it.K = (int32_t)K;
    it.P = (int32_t)ceil_div(K, AFF_TILE_K);
    it.units = (int32_t)ceil_div(N, RB);
    it.out_f32 = out_f32 ? 1 : 0;
    const int64_t cap = (int64_t)cus * affine_gemv_wgs_per_cu();
    const int grid = (int)(it.units < cap ? it.units : cap);
    return launch_ag_fmt<false>(nullptr, nullptr, it, grid, K, bits, group, bf16_scales, s);
}

hipError_t launch_affine_gemv_list(const WorkItem *items, const WorkStart *starts, int grid,
                                   int64_t kmax, int bits, int group, bool bf16_scales,
                                   hipStream_t s) {
    WorkItem none{};
    return launch_ag_fmt<true>(items, starts, none, grid, kmax, bits, group, bf16_scales, s);
}

}  // namespace qg
