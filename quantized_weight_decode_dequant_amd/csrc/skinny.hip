// Skinny products Y[M, N] = X[M, K] W^T for M = 1..32 activation rows against
// weights streamed once per call: the verification pass of a 16-32 token
// draft (Uzu page, fange-kb.cn, section "Producing several tokens from one
// model pass": sixteen candidate rows give the matrix units sixteen rows of
// work instead of one).  Both kernels run on the gfx950 MFMA units with the
// 16x16x32 shapes, whose B operand (lane l: 8 consecutive k of column l & 15,
// k-slice l >> 4) is exactly one packed weight slot (see qg_internal.h).
//
// Q4 (bf16 X): each packed word becomes the bf16x8 operand (128 + q); one
// MFMA pair covers one group of 64, its fp32 result is scaled per (row n,
// group) on the VALU: acc += s * C + (b - 128 s) * sum_{k in g} X[m, k].
// Q8 (int8 X from the Hadamard quantizer): one i8 MFMA per group of 32 gives
// the exact int32 group partial; acc += sw * float(partial) (exact
// conversion, |partial| <= 32 * 127^2), then y = sx[m] * acc.
//
// Work split: a workgroup of 4 waves owns a unit of 4 * RPW consecutive
// rowblocks (each wave RPW rowblocks, sharing its A operands across them)
// and walks K in chunks of KC tiles; each chunk of X is staged into LDS
// (rows padded by 16 bytes so the 16 A-operand rows hit distinct banks) and
// shared by the 4 waves.  The Q4 kernel also runs over a device work list of
// independent matrices (one launch for a whole verification pass).
#include "qg_internal.h"

namespace qg {

constexpr int SK_WAVES = 4;
constexpr int SK_THREADS = SK_WAVES * 64;

template <int MT, int KC, int RPW>
__device__ __forceinline__ void sk_q4_unit(const WorkItem &it, int unit, int M, uint16_t *xl,
                                           float *xs, int tid, const Q4Consts &magic) {
    constexpr int MP = MT * 16;
    constexpr int RS = KC * 128 + 8;  // LDS row stride in bf16
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), kg = lane >> 4;
    const int P = it.P, K = it.K, N = it.N;
    const int nrb = (N + RB - 1) / RB;
    const int rb0 = unit * (SK_WAVES * RPW) + wave * RPW;
    const uint16_t *X = reinterpret_cast<const uint16_t *>(it.x);
    f32x4_t acc[RPW][MT];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[r][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int pc = 0; pc < P; pc += KC) {
        const int nt = min(KC, P - pc);
        // this chunk's weight slots (clamped indices: always in bounds)
        u32x4_t c[KC][RPW];
        u32x2_t sb[KC][RPW];
#pragma unroll
        for (int j = 0; j < KC; ++j)
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                const int rb = min(rb0 + r, nrb - 1);
                const int p = min(pc + j, P - 1);
                const uint8_t *tb = it.packed + ((size_t)rb * P + p) * Q4_TILE_BYTES;
                c[j][r] = ld_nt(reinterpret_cast<const u32x4_t *>(tb) + lane);
                sb[j][r] = ld_nt(reinterpret_cast<const u32x2_t *>(tb + 1024) + (lane & 15));
            }
        __syncthreads();  // the previous chunk's LDS reads are done
        {
            constexpr int TOT = MP * KC * 16;  // uint4 per chunk
            constexpr int U = (TOT + SK_THREADS - 1) / SK_THREADS;
            const int k0 = pc * 128;
            uint4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = tid + u * SK_THREADS;
                const int m = i / (KC * 16), c8 = i % (KC * 16);
                const int k = k0 + c8 * 8;
                v[u] = (i < TOT && m < M && k < K)
                           ? *reinterpret_cast<const uint4 *>(X + (size_t)m * K + k)
                           : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = tid + u * SK_THREADS;
                const int m = i / (KC * 16), c8 = i % (KC * 16);
                if (i < TOT) *reinterpret_cast<uint4 *>(xl + m * RS + c8 * 8) = v[u];
            }
        }
        __syncthreads();
        for (int i = tid; i < 2 * KC * MP; i += SK_THREADS) {
            const int g = i / MP, m = i % MP;
            const uint4 *rr = reinterpret_cast<const uint4 *>(xl + m * RS + g * 64);
            float sum = 0.f;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint4 v = rr[q];
                sum += bf16_lo(v.x) + bf16_hi(v.x) + bf16_lo(v.y) + bf16_hi(v.y) + bf16_lo(v.z) +
                       bf16_hi(v.z) + bf16_lo(v.w) + bf16_hi(v.w);
            }
            xs[i] = sum;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            if (j < nt) {
                bf16x8_t A[MT][4];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const uint16_t *ar = xl + (16 * mt + (lane & 15)) * RS + j * 128 + 8 * kg;
#pragma unroll
                    for (int q = 0; q < 4; ++q) A[mt][q] = *reinterpret_cast<const bf16x8_t *>(ar + 32 * q);
                }
                f32x4_t xs0[MT], xs1[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    xs0[mt] = *reinterpret_cast<const f32x4_t *>(xs + (2 * j) * MP + 16 * mt + 4 * kg);
                    xs1[mt] = *reinterpret_cast<const f32x4_t *>(xs + (2 * j + 1) * MP + 16 * mt + 4 * kg);
                }
#pragma unroll
                for (int r = 0; r < RPW; ++r) {
                    if (rb0 + r < nrb) {
                        bf16x8_t B[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) B[q] = q4_word_to_bf16x8(c[j][r][q], magic);
                        const float s0 = f16_lo(sb[j][r][0]), b0 = f16_hi(sb[j][r][0]);
                        const float s1 = f16_lo(sb[j][r][1]), b1 = f16_hi(sb[j][r][1]);
                        const float bb0 = fmaf(-128.f, s0, b0), bb1 = fmaf(-128.f, s1, b1);
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
                            f32x4_t C0 = {0.f, 0.f, 0.f, 0.f}, C1 = {0.f, 0.f, 0.f, 0.f};
                            C0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][0], B[0], C0, 0, 0, 0);
                            C0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][1], B[1], C0, 0, 0, 0);
                            C1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][2], B[2], C1, 0, 0, 0);
                            C1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][3], B[3], C1, 0, 0, 0);
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                float a = acc[r][mt][i];
                                a = fmaf(s0, C0[i], a);
                                a = fmaf(bb0, xs0[mt][i], a);
                                a = fmaf(s1, C1[i], a);
                                a = fmaf(bb1, xs1[mt][i], a);
                                acc[r][mt][i] = a;
                            }
                        }
                    }
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int n = (rb0 + r) * RB + (lane & 15);
        if (rb0 + r < nrb && n < N) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = 16 * mt + 4 * kg + i;
                    if (m < M) {
                        if (it.out_f32)
                            reinterpret_cast<float *>(it.y)[(size_t)m * N + n] = acc[r][mt][i];
                        else
                            reinterpret_cast<uint16_t *>(it.y)[(size_t)m * N + n] =
                                f32_to_bf16(acc[r][mt][i]);
                    }
                }
        }
    }
}

template <int MT, int KC, int RPW>
__global__ void __launch_bounds__(SK_THREADS)
q4_skinny_kernel(const WorkItem *__restrict__ items, const WorkStart *__restrict__ starts,
                 WorkItem single, int M) {
    constexpr int MP = MT * 16;
    constexpr int RS = KC * 128 + 8;
    __shared__ __attribute__((aligned(16))) uint16_t xl[MP * RS];
    __shared__ __attribute__((aligned(16))) float xs[2 * KC * MP];  // [group-in-chunk][m]
    const int tid = threadIdx.x;
    const Q4Consts magic = q4_consts();
    if (items == nullptr) {
        for (int u = blockIdx.x; u < single.units; u += gridDim.x)
            sk_q4_unit<MT, KC, RPW>(single, u, M, xl, xs, tid, magic);
        return;
    }
    const WorkStart s = starts[blockIdx.x], e = starts[blockIdx.x + 1];
    int i = s.item, u = s.unit, loaded = -1;
    WorkItem it;
    while (i < e.item || (i == e.item && u < e.unit)) {
        if (i != loaded) {
            it = items[i];
            loaded = i;
        }
        sk_q4_unit<MT, KC, RPW>(it, u, M, xl, xs, tid, magic);
        if (++u == it.units) {
            ++i;
            u = 0;
        }
    }
}

// out_mode: 0 = bf16, 1 = fp32, 2 = int32 group partials [M][N][K/32]
template <int MT, int KC>
__global__ void __launch_bounds__(SK_THREADS)
q8_skinny_kernel(const uint8_t *__restrict__ packed, const int8_t *__restrict__ X,
                 const float *__restrict__ x_scales, void *__restrict__ Y, int M, int N, int K,
                 int P, int nrb, int out_mode) {
    constexpr int MP = MT * 16;
    constexpr int RS = KC * 128 + 16;  // LDS row stride in bytes
    __shared__ __attribute__((aligned(16))) int8_t xl[MP * RS];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), kg = lane >> 4;
    const int G = K / 32;
    const int items = (nrb + SK_WAVES - 1) / SK_WAVES;
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int rb = item * SK_WAVES + wave;
        const bool active = rb < nrb;
        const uint8_t *base = packed + (size_t)(active ? rb : nrb - 1) * P * Q8_TILE_BYTES;
        const int n = rb * RB + (lane & 15);
        f32x4_t acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int pc = 0; pc < P; pc += KC) {
            const int nt = min(KC, P - pc);
            u32x4_t c0[KC], c1[KC];
            u32x2_t sc[KC];
#pragma unroll
            for (int j = 0; j < KC; ++j) {
                const uint8_t *tb = base + (size_t)min(pc + j, P - 1) * Q8_TILE_BYTES;
                c0[j] = ld_nt(reinterpret_cast<const u32x4_t *>(tb) + lane);
                c1[j] = ld_nt(reinterpret_cast<const u32x4_t *>(tb + 1024) + lane);
                sc[j] = ld_nt(reinterpret_cast<const u32x2_t *>(tb + 2048) + (lane & 15));
            }
            __syncthreads();
            {
                constexpr int TOT = MP * KC * 8;  // uint4 per chunk
                constexpr int U = (TOT + SK_THREADS - 1) / SK_THREADS;
                const int k0 = pc * 128;
                uint4 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int i = tid + u * SK_THREADS;
                    const int m = i / (KC * 8), c16 = i % (KC * 8);
                    const int k = k0 + c16 * 16;
                    v[u] = (i < TOT && m < M && k < K)
                               ? *reinterpret_cast<const uint4 *>(X + (size_t)m * K + k)
                               : make_uint4(0u, 0u, 0u, 0u);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int i = tid + u * SK_THREADS;
                    const int m = i / (KC * 8), c16 = i % (KC * 8);
                    if (i < TOT) *reinterpret_cast<uint4 *>(xl + m * RS + c16 * 16) = v[u];
                }
            }
            __syncthreads();
            if (active) {
#pragma unroll
                for (int j = 0; j < KC; ++j) {
                    if (j < nt) {
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            const u32x4_t ch = (g4 < 2) ? c0[j] : c1[j];
                            const int gg = g4 & 1;
                            const long bop = (long)(((unsigned long)ch[2 * gg + 1] << 32) | ch[2 * gg]);
                            const unsigned swbits = (g4 < 2) ? sc[j][0] : sc[j][1];
                            const float sw = (g4 & 1) ? f16_hi(swbits) : f16_lo(swbits);
                            const int g = (pc + j) * 4 + g4;
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt) {
                                const int8_t *ar = xl + (16 * mt + (lane & 15)) * RS + j * 128 + 32 * g4 + 8 * kg;
                                const long aop = *reinterpret_cast<const long *>(ar);
                                i32x4_t C = {0, 0, 0, 0};
                                C = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop, C, 0, 0, 0);
                                if (out_mode == 2) {
                                    if (g < G) {
#pragma unroll
                                        for (int i = 0; i < 4; ++i) {
                                            const int m = 16 * mt + 4 * kg + i;
                                            if (m < M && n < N)
                                                reinterpret_cast<int32_t *>(Y)[((size_t)m * N + n) * G + g] = C[i];
                                        }
                                    }
                                } else {
#pragma unroll
                                    for (int i = 0; i < 4; ++i) acc[mt][i] = fmaf(sw, (float)C[i], acc[mt][i]);
                                }
                            }
                        }
                    }
                }
            }
        }
        if (active && out_mode != 2) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = 16 * mt + 4 * kg + i;
                    if (m < M && n < N) {
                        const float v = x_scales[m] * acc[mt][i];
                        if (out_mode == 1)
                            reinterpret_cast<float *>(Y)[(size_t)m * N + n] = v;
                        else
                            reinterpret_cast<uint16_t *>(Y)[(size_t)m * N + n] = f32_to_bf16(v);
                    }
                }
        }
    }
}

static inline int sk_units(int64_t N, int rowblocks_per_unit) {
    return (int)ceil_div(ceil_div(N, RB), rowblocks_per_unit);
}

static inline int min_grid(int units, int cap) { return units < cap ? units : cap; }

hipError_t launch_q4_skinny(const uint8_t *packed, const uint16_t *X, void *Y, int64_t M,
                            int64_t N, int64_t K, bool out_f32, int cus, hipStream_t s) {
    WorkItem it{};
    it.packed = packed;
    it.x = X;
    it.y = Y;
    it.N = (int32_t)N;
    it.K = (int32_t)K;
    it.P = (int32_t)ceil_div(K, Q4_TILE_K);
    it.out_f32 = out_f32 ? 1 : 0;
    if (M <= 16) {
        it.units = sk_units(N, SK_ROWBLOCKS_M16);
        hipLaunchKernelGGL((q4_skinny_kernel<1, 8, SK_ROWBLOCKS_M16 / SK_WAVES>),
                           dim3(min_grid(it.units, cus * 4)), dim3(SK_THREADS), 0, s,
                           (const WorkItem *)nullptr, (const WorkStart *)nullptr, it, (int)M);
    } else {
        it.units = sk_units(N, SK_ROWBLOCKS_M32);
        hipLaunchKernelGGL((q4_skinny_kernel<2, 4, SK_ROWBLOCKS_M32 / SK_WAVES>),
                           dim3(min_grid(it.units, cus * 4)), dim3(SK_THREADS), 0, s,
                           (const WorkItem *)nullptr, (const WorkStart *)nullptr, it, (int)M);
    }
    return hipGetLastError();
}

hipError_t launch_q4_skinny_list(const WorkItem *items, const WorkStart *starts, int grid,
                                 int64_t M, hipStream_t s) {
    WorkItem none{};
    if (M <= 16)
        hipLaunchKernelGGL((q4_skinny_kernel<1, 8, SK_ROWBLOCKS_M16 / SK_WAVES>), dim3(grid),
                           dim3(SK_THREADS), 0, s, items, starts, none, (int)M);
    else
        hipLaunchKernelGGL((q4_skinny_kernel<2, 4, SK_ROWBLOCKS_M32 / SK_WAVES>), dim3(grid),
                           dim3(SK_THREADS), 0, s, items, starts, none, (int)M);
    return hipGetLastError();
}

hipError_t launch_q8_skinny(const uint8_t *packed, const int8_t *X, const float *x_scales,
                            void *Y, int64_t M, int64_t N, int64_t K, int out_mode, int cus,
                            hipStream_t s) {
    const int P = (int)ceil_div(K, Q8_TILE_K);
    const int nrb = (int)ceil_div(N, RB);
    const int units = (nrb + SK_WAVES - 1) / SK_WAVES;
    if (M <= 16) {
        hipLaunchKernelGGL((q8_skinny_kernel<1, 8>), dim3(min_grid(units, cus * 4)), dim3(SK_THREADS),
                           0, s, packed, X, x_scales, Y, (int)M, (int)N, (int)K, P, nrb, out_mode);
    } else {
        hipLaunchKernelGGL((q8_skinny_kernel<2, 4>), dim3(min_grid(units, cus * 4)), dim3(SK_THREADS),
                           0, s, packed, X, x_scales, Y, (int)M, (int)N, (int)K, P, nrb, out_mode);
    }
    return hipGetLastError();
}

}  // namespace qg
