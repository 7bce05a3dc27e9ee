// Block-diagonal randomized Hadamard-32 rotation followed by per-row int8
// quantization of the activations (Uzu page, fange-kb.cn, section "How Uzu
// optimizes bytes and tokens per pass": +-1 Hadamard entries and one global
// scale, random sign flips applied before the mixing, independent blocks of
// 32 chosen to match a 32-wide SIMD group, fully invertible; activations are
// quantized to 8 bits on the fly so verification runs on the int8 matrix
// path).
//
// One workgroup per activation row: 8 waves for rows of up to 12288 (one
// round, three 16-block units per wave), 16 for longer ones.  Four lanes own one
// block of 32: lane part p holds elements 8p .. 8p + 7, so the first three
// butterfly stages (index bits 0, 1, 2) are register adds and subtracts and
// the last two (bits 3, 4) exchange with the lanes p ^ 1 and p ^ 2 of the
// same quad through DPP moves.  Stages run in index-bit order and the lower
// index of each pair takes a + c, the upper a - c, so after the five stages
// the lane holds z_i = sum_j (-1)^popcount(i & j) d_j x_j (Sylvester
// order).  The sums are carried in fp64, where a signed sum of 32 bf16 values
// is exact for activations of ordinary range, so the quantization decision
// sees the exact z.  A row of up to 24576 elements is loaded once, with every
// load issued up front, and its z kept in registers; the row maximum amax =
// max |z| is reduced within each wave by DPP moves and across the waves
// through LDS.  Each code is round-half-even(z * 127 / amax) of the
// correctly rounded fp64 quotient: it is taken from the product z * (127 /
// amax) unless that product lies within 1e-9 of a rounding boundary (its
// error is below 1e-13), in which case the quotient is computed by a true
// division (a branch taken only by waves with such an element).  Since |z|
// <= amax, both give codes within [-127, 127]: no clamp is needed.  Longer
// rows are processed in rounds of 24576 and recomputed from x for the
// second pass.
#include "qg_internal.h"

namespace qg {

constexpr int HQ_R = 3;  // 16-block units per wave per round (512 k each)

// Exchange with the lane p ^ S of the quad (S = 1 or 2), by DPP quad_perm.
template <int S>
__device__ __forceinline__ double quad_xor(double v) {
    constexpr int ctrl = S == 1 ? 0xB1 : 0x4E;  // [1,0,3,2] / [2,3,0,1]
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    const int lo = __builtin_amdgcn_mov_dpp((int)(unsigned)u, ctrl, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(unsigned)(u >> 32), ctrl, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

// v moved across lanes by the DPP control ctrl (both 32-bit halves).
template <int CTRL>
__device__ __forceinline__ double dpp64(double v) {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    const int lo = __builtin_amdgcn_mov_dpp((int)(unsigned)u, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(unsigned)(u >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

// The largest v of the wave, in every lane: within each row of 16 lanes by
// DPP moves (quad exchanges, then rotations by 4 and 8), then the four row
// maxima read from lanes 0, 16, 32 and 48.  VALU work only, no trip through
// the LDS crossbar per step.
__device__ __forceinline__ double wave_max(double v) {
    v = fmax(v, dpp64<0xB1>(v));   // quad_perm [1,0,3,2]
    v = fmax(v, dpp64<0x4E>(v));   // quad_perm [2,3,0,1]
    v = fmax(v, dpp64<0x124>(v));  // row_ror:4
    v = fmax(v, dpp64<0x128>(v));  // row_ror:8
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    double r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned lo = __builtin_amdgcn_readlane((unsigned)u, 16 * i);
        const unsigned hi = __builtin_amdgcn_readlane((unsigned)(u >> 32), 16 * i);
        r[i] = __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
    }
    return fmax(fmax(r[0], r[1]), fmax(r[2], r[3]));
}

// The five butterfly stages over this lane's 8 elements (part p of the block).
__device__ __forceinline__ void fwht32_oct(double z[8], int p) {
#pragma unroll
    for (int s = 1; s < 8; s <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (!(e & s)) {
                const double a = z[e], c = z[e + s];
                z[e] = a + c;
                z[e + s] = a - c;
            }
    // the upper index of a pair takes o - z, the lower z + o: one fma with
    // z * (-1 or +1) + o, rounded once like the add or subtract it replaces
    const double sg1 = (p & 1) ? -1.0 : 1.0, sg2 = (p & 2) ? -1.0 : 1.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = fma(z[e], sg1, quad_xor<1>(z[e]));
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = fma(z[e], sg2, quad_xor<2>(z[e]));
}

// Load and transform this wave's units of one round.  Unit u covers blocks
// 16u .. 16u + 15, lane l takes block 16u + (l >> 2), part l & 3.  Buffer
// loads past the row read as zero.
template <int HQ_WAVES>
__device__ __forceinline__ void hq_round(__amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rsg,
                                         int nunit, int round, int wave, int lane,
                                         double z[HQ_R][8]) {
    const int p = lane & 3;
    u32x4_t xv[HQ_R];
    u32x2_t sv[HQ_R];
#pragma unroll
    for (int i = 0; i < HQ_R; ++i) {
        const int u = (round * HQ_R + i) * HQ_WAVES + wave;
        const unsigned k = 32u * (16u * (unsigned)u + (lane >> 2)) + 8u * p;
        if (u < nunit) {  // uniform
            xv[i] = buf_ld_x4(rx, 2u * k, 0);
            sv[i] = buf_ld_x2(rsg, k, 0);
        } else {
            xv[i] = u32x4_t{0u, 0u, 0u, 0u};
            sv[i] = u32x2_t{0u, 0u};
        }
    }
#pragma unroll
    for (int i = 0; i < HQ_R; ++i) {
        if ((round * HQ_R + i) * HQ_WAVES + wave >= nunit) {  // uniform
#pragma unroll
            for (int e = 0; e < 8; ++e) z[i][e] = 0.0;
            continue;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const unsigned w = xv[i][e >> 1];
            const float x = (e & 1) ? bf16_hi(w) : bf16_lo(w);
            const int d = (int)(int8_t)((sv[i][e >> 2] >> (8 * (e & 3))) & 0xFFu);
            z[i][e] = (double)d * (double)x;
        }
        fwht32_oct(z[i], p);
    }
}

template <int HQ_WAVES>
__global__ void __launch_bounds__(HQ_WAVES * 64)
had32_quant_kernel(const uint16_t *__restrict__ X, const int8_t *__restrict__ signs, int K,
                   int8_t *__restrict__ Xq, float *__restrict__ x_scales, double denom) {
    __shared__ double wmax[HQ_WAVES];
    const int m = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nblk = K / 32;
    const int nunit = (nblk + 15) / 16;
    const int nround = (nunit + HQ_WAVES * HQ_R - 1) / (HQ_WAVES * HQ_R);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + (size_t)m * K, 2u * (unsigned)K);
    const __amdgpu_buffer_rsrc_t rsg = make_rsrc(signs, (unsigned)K);
    double z[HQ_R][8];
    double amax = 0.0;
#pragma unroll 1
    for (int r = 0; r < nround; ++r) {
        hq_round<HQ_WAVES>(rx, rsg, nunit, r, wave, lane, z);
#pragma unroll
        for (int i = 0; i < HQ_R; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmax(amax, fabs(z[i][e]));
    }
    // row maximum: wave, then across waves
    amax = wave_max(amax);
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    amax = 0.0;
#pragma unroll
    for (int w = 0; w < HQ_WAVES; ++w) amax = fmax(amax, wmax[w]);
    // amax is 0 or at least the smallest bf16 magnitude (2^-133), so s is finite
    const double s = amax > 0.0 ? 127.0 / amax : 0.0;

    int8_t *qr = Xq + (size_t)m * K;
#pragma unroll 1
    for (int r = nround - 1; r >= 0; --r) {
        // the last round is still in registers
        if (r != nround - 1) hq_round<HQ_WAVES>(rx, rsg, nunit, r, wave, lane, z);
#pragma unroll
        for (int i = 0; i < HQ_R; ++i) {
            const int u = (r * HQ_R + i) * HQ_WAVES + wave;
            const int b = 16 * u + (lane >> 2);
            if (u >= nunit) break;  // uniform
            // codes from the product with 127 / amax; only when some lane of
            // the wave meets a product within 1e-9 of a rounding boundary do
            // the flagged elements take the true quotient (one uniform branch)
            double q[8];
            bool near = false;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double p = z[i][e] * s;
                q[e] = rint(p);
                near = near || fabs(p - q[e]) > 0.5 - 1e-9;
            }
            if (__any(near)) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const double p = z[i][e] * s;
                    if (fabs(p - rint(p)) > 0.5 - 1e-9) q[e] = rint(z[i][e] * 127.0 / amax);
                }
            }
            unsigned packed[2] = {0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                packed[e >> 2] |= ((unsigned)(int)q[e] & 0xFFu) << (8 * (e & 3));
            if (b < nblk)
                *reinterpret_cast<u32x2_t *>(qr + 32 * b + 8 * (lane & 3)) =
                    u32x2_t{packed[0], packed[1]};
        }
    }
    if (tid == 0) x_scales[m] = amax > 0.0 ? (float)(amax / denom) : 0.f;
}

hipError_t launch_had32_quant(const uint16_t *X, const int8_t *signs, int64_t M, int64_t K,
                              int8_t *Xq, float *x_scales, double denom, hipStream_t s) {
    // 8 waves take a row of up to 8 * HQ_R units (12288 k) in one round and
    // ran 16 x 4096 in 3.23 us and 16 x 12288 in 4.68 us against 3.93 and
    // 4.95 with 16 waves (4 waves: 3.27 / 6.11, 12: 3.39 / 4.75); longer rows
    // take 16 waves, so that 24576 k is still one round
    if (K <= 8 * HQ_R * 512)
        hipLaunchKernelGGL((had32_quant_kernel<8>), dim3((unsigned)M), dim3(8 * 64), 0, s, X,
                           signs, (int)K, Xq, x_scales, denom);
    else
        hipLaunchKernelGGL((had32_quant_kernel<16>), dim3((unsigned)M), dim3(16 * 64), 0, s, X,
                           signs, (int)K, Xq, x_scales, denom);
    return hipGetLastError();
}

}  // namespace qg
