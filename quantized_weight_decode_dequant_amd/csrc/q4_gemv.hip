// Decode GEMV, one activation row, 4-bit asymmetric group-64 weights:
//     y[n] = sum_g ( s[n,g] * sum_{k in g} q[n,k] x[k]  +  b[n,g] * sum_{k in g} x[k] )
// which is sum_k (s*q + b) x with the weight dequantized in registers and
// never stored ("MLX Runner: An Inference Engine You Can Read", section
// "Architecture: one command buffer per token": weight = scale x code + bias;
// Uzu page, section "Why batch-one decoding is memory-bound": every weight is
// streamed once with about one multiply-add).
//
// Work split.  A workgroup owns one rowblock (16 rows) at a time and loops
// over rowblocks (grid-stride); its waves split the rowblock's 128-k tiles.
// Each lane reads one 16-byte slot per tile (4 words = 32 codes of one row),
// one 64-lane load covers 16 rows x 128 k = 1 KB contiguous.  x is staged in
// LDS once per workgroup together with per-(tile, group, k-slice) partial
// sums of x, which carry the bias term.
//
// Arithmetic per word: (w >> 4j) & 0x000F000F | 0x43004300 turns two codes
// into the bf16 pair (128 + q, 128 + q'), exact; v_dot2_f32_bf16 multiplies
// it with the matching x pair and adds in fp32.  The 128 offset is removed
// with the group's x partial sum: s * sum (128 + q) x + (b - 128 s) * sum x.
// Lanes of one row (k-slices 0..3) are summed with two xor shuffles, then the
// waves through LDS, in a fixed order (deterministic).
#include "qg_internal.h"

namespace qg {

template <int WAVES, int TPW>
__global__ void __launch_bounds__(WAVES * 64)
q4_gemv_kernel(const uint8_t *__restrict__ packed, const uint16_t *__restrict__ x,
               void *__restrict__ y, int N, int K, int P, int nrb, int out_f32) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned *xl = reinterpret_cast<unsigned *>(smem);          // bf16 pairs [P*64]
    float *xsum = reinterpret_cast<float *>(smem + (size_t)P * 256);  // [P*8]
    float *red = xsum + P * 8;                                   // [2][WAVES][16]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // stage x (zero past K) and the per-(tile, group, k-slice) x sums
    const int nx4 = K / 8;
    for (int i = tid; i < P * 16; i += WAVES * 64) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (i < nx4) v = reinterpret_cast<const uint4 *>(x)[i];
        reinterpret_cast<uint4 *>(xl)[i] = v;
    }
    __syncthreads();
    for (int i = tid; i < P * 8; i += WAVES * 64) {
        const int p = i >> 3, t = (i >> 2) & 1, kg = i & 3;
        float s = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const unsigned *b = xl + p * 64 + 32 * t + 16 * h + 4 * kg;
#pragma unroll
            for (int d = 0; d < 4; ++d) s += bf16_lo(b[d]) + bf16_hi(b[d]);
        }
        xsum[i] = s;
    }
    __syncthreads();

    const int kg = lane >> 4;
    int par = 0;
    for (int rb = blockIdx.x; rb < nrb; rb += gridDim.x) {
        const uint8_t *base = packed + (size_t)rb * P * Q4_TILE_BYTES;
        float acc = 0.f;
        for (int p0 = wave; p0 < P; p0 += WAVES * TPW) {
            u32x4_t c[TPW];
            u32x2_t sb[TPW];
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int p = p0 + j * WAVES;
                if (p < P) {
                    const uint8_t *tb = base + (size_t)p * Q4_TILE_BYTES;
                    c[j] = ld_nt(reinterpret_cast<const u32x4_t *>(tb) + lane);
                    sb[j] = ld_nt(reinterpret_cast<const u32x2_t *>(tb + 1024) + (lane & 15));
                }
            }
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int p = p0 + j * WAVES;
                if (p < P) {
                    const uint4 *xp = reinterpret_cast<const uint4 *>(xl) + 16 * p + kg;
                    const uint4 xa0 = xp[0], xb0 = xp[4], xa1 = xp[8], xb1 = xp[12];
                    float d0 = 0.f, d1 = 0.f;
                    d0 = dot2_bf16(q4_pair_bias128<0>(c[j][0]), xa0.x, d0);
                    d0 = dot2_bf16(q4_pair_bias128<1>(c[j][0]), xa0.y, d0);
                    d0 = dot2_bf16(q4_pair_bias128<2>(c[j][0]), xa0.z, d0);
                    d0 = dot2_bf16(q4_pair_bias128<3>(c[j][0]), xa0.w, d0);
                    d0 = dot2_bf16(q4_pair_bias128<0>(c[j][1]), xb0.x, d0);
                    d0 = dot2_bf16(q4_pair_bias128<1>(c[j][1]), xb0.y, d0);
                    d0 = dot2_bf16(q4_pair_bias128<2>(c[j][1]), xb0.z, d0);
                    d0 = dot2_bf16(q4_pair_bias128<3>(c[j][1]), xb0.w, d0);
                    d1 = dot2_bf16(q4_pair_bias128<0>(c[j][2]), xa1.x, d1);
                    d1 = dot2_bf16(q4_pair_bias128<1>(c[j][2]), xa1.y, d1);
                    d1 = dot2_bf16(q4_pair_bias128<2>(c[j][2]), xa1.z, d1);
                    d1 = dot2_bf16(q4_pair_bias128<3>(c[j][2]), xa1.w, d1);
                    d1 = dot2_bf16(q4_pair_bias128<0>(c[j][3]), xb1.x, d1);
                    d1 = dot2_bf16(q4_pair_bias128<1>(c[j][3]), xb1.y, d1);
                    d1 = dot2_bf16(q4_pair_bias128<2>(c[j][3]), xb1.z, d1);
                    d1 = dot2_bf16(q4_pair_bias128<3>(c[j][3]), xb1.w, d1);
                    const float s0 = f16_lo(sb[j][0]), b0 = f16_hi(sb[j][0]);
                    const float s1 = f16_lo(sb[j][1]), b1 = f16_hi(sb[j][1]);
                    const float xs0 = xsum[p * 8 + kg], xs1 = xsum[p * 8 + 4 + kg];
                    acc = fmaf(s0, d0, acc);
                    acc = fmaf(fmaf(-128.f, s0, b0), xs0, acc);
                    acc = fmaf(s1, d1, acc);
                    acc = fmaf(fmaf(-128.f, s1, b1), xs1, acc);
                }
            }
        }
        acc += __shfl_xor(acc, 16);
        acc += __shfl_xor(acc, 32);
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

hipError_t launch_q4_gemv(const uint8_t *packed, const uint16_t *x, void *y, int64_t N,
                          int64_t K, bool out_f32, int cus, hipStream_t s) {
    constexpr int WAVES = 4, TPW = 8;
    const int P = (int)ceil_div(K, Q4_TILE_K);
    const int nrb = (int)ceil_div(N, RB);
    const size_t lds = (size_t)P * 256 + (size_t)P * 32 + 2 * WAVES * 16 * 4;
    const int grid = (int)(nrb < (int64_t)cus * 8 ? nrb : (int64_t)cus * 8);
    hipLaunchKernelGGL((q4_gemv_kernel<WAVES, TPW>), dim3(grid), dim3(WAVES * 64), lds, s,
                       packed, x, y, (int)N, (int)K, P, nrb, out_f32 ? 1 : 0);
    return hipGetLastError();
}

}  // namespace qg
