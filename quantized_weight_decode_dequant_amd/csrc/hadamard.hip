// Block-diagonal randomized Hadamard-32 rotation followed by per-row int8
// quantization of the activations (Uzu page, fange-kb.cn, section "How Uzu
// optimizes bytes and tokens per pass": +-1 Hadamard entries and one global
// scale, random sign flips applied before the mixing, independent blocks of
// 32 chosen to match a 32-wide SIMD group, fully invertible; activations are
// quantized to 8 bits on the fly so verification runs on the int8 matrix
// path).
//
// One workgroup of 1024 threads per activation row.  Each 16-lane quarter
// of a wavefront owns one block of 32: lane p holds elements 2p and 2p + 1,
// so the first butterfly stage (index bit 0) is a register add/subtract and
// the other four (bits 1..4) exchange across lanes p ^ 1, 2, 4, 8.  After
// the five stages the lane holds z_i = sum_j (-1)^popcount(i & j) d_j x_j
// (Sylvester order) for its two i.  The sums are carried in fp64, where a
// signed sum of 32 bf16 values is exact for activations of ordinary range,
// so the quantization decision sees the exact z.  A row of up to 24576
// elements is loaded once with every load issued up front and its z kept in
// registers; the row maximum amax = max |z| is reduced through LDS and the
// same registers are quantized to round-half-even(z * 127 / amax) (fp64
// division, correctly rounded).  Longer rows are processed in rounds of
// 24576 and recomputed from x for the second pass.
#include "qg_internal.h"

namespace qg {

constexpr int HQ_THREADS = 1024;
constexpr int HQ_WAVES = HQ_THREADS / 64;
constexpr int HQ_R = 12;  // 4-block units per wave per round (24576 k per round)

// z of this lane's two elements of a block: v0 = d_2p x_2p, v1 = d_2p+1 x_2p+1.
__device__ __forceinline__ void fwht32_pair(double &v0, double &v1, int p) {
    const double s0 = v0 + v1, s1 = v0 - v1;
    v0 = s0;
    v1 = s1;
#pragma unroll
    for (int s = 1; s < 16; s <<= 1) {
        const double o0 = __shfl_xor(v0, s), o1 = __shfl_xor(v1, s);
        v0 = (p & s) ? (o0 - v0) : (v0 + o0);
        v1 = (p & s) ? (o1 - v1) : (v1 + o1);
    }
}

// Load and transform one round: unit u = round * HQ_WAVES * HQ_R + wave +
// HQ_WAVES * i covers blocks 4u .. 4u + 3; lane l takes block 4u + (l >> 4).
__device__ __forceinline__ void hq_round(const uint16_t *xr, const int8_t *signs, int nblk,
                                         int round, int wave, int lane, double z[HQ_R][2],
                                         bool ok[HQ_R]) {
    const int p = lane & 15;
    unsigned xv[HQ_R];
    unsigned short sv[HQ_R];
#pragma unroll
    for (int i = 0; i < HQ_R; ++i) {
        const int b = 4 * ((round * HQ_R + i) * HQ_WAVES + wave) + (lane >> 4);
        ok[i] = b < nblk;
        const int k = 32 * b + 2 * p;
        xv[i] = ok[i] ? *reinterpret_cast<const unsigned *>(xr + k) : 0u;
        sv[i] = ok[i] ? *reinterpret_cast<const unsigned short *>(signs + k) : (unsigned short)0;
    }
#pragma unroll
    for (int i = 0; i < HQ_R; ++i) {
        const double d0 = (double)(int8_t)(sv[i] & 0xFF), d1 = (double)(int8_t)(sv[i] >> 8);
        z[i][0] = d0 * (double)bf16_lo(xv[i]);
        z[i][1] = d1 * (double)bf16_hi(xv[i]);
        fwht32_pair(z[i][0], z[i][1], p);
    }
}

__global__ void __launch_bounds__(HQ_THREADS)
had32_quant_kernel(const uint16_t *__restrict__ X, const int8_t *__restrict__ signs, int K,
                   int8_t *__restrict__ Xq, float *__restrict__ x_scales, double denom) {
    __shared__ double wmax[HQ_WAVES];
    const int m = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p = lane & 15;
    const int nblk = K / 32;
    const int nround = (nblk + 4 * HQ_WAVES * HQ_R - 1) / (4 * HQ_WAVES * HQ_R);
    const uint16_t *xr = X + (size_t)m * K;
    double z[HQ_R][2];
    bool ok[HQ_R];
    double amax = 0.0;
#pragma unroll 1
    for (int r = 0; r < nround; ++r) {
        hq_round(xr, signs, nblk, r, wave, lane, z, ok);
#pragma unroll
        for (int i = 0; i < HQ_R; ++i)
            if (ok[i]) amax = fmax(amax, fmax(fabs(z[i][0]), fabs(z[i][1])));
    }
    // row maximum: wave, then across waves
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) amax = fmax(amax, __shfl_xor(amax, s));
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    amax = 0.0;
#pragma unroll
    for (int w = 0; w < HQ_WAVES; ++w) amax = fmax(amax, wmax[w]);

    int8_t *qr = Xq + (size_t)m * K;
#pragma unroll 1
    for (int r = nround - 1; r >= 0; --r) {
        // the last round is still in registers
        if (r != nround - 1) hq_round(xr, signs, nblk, r, wave, lane, z, ok);
#pragma unroll
        for (int i = 0; i < HQ_R; ++i) {
            if (!ok[i]) continue;
            double q0 = 0.0, q1 = 0.0;
            if (amax > 0.0) {
                q0 = fmin(fmax(rint(z[i][0] * 127.0 / amax), -127.0), 127.0);
                q1 = fmin(fmax(rint(z[i][1] * 127.0 / amax), -127.0), 127.0);
            }
            const int b = 4 * ((r * HQ_R + i) * HQ_WAVES + wave) + (lane >> 4);
            const unsigned short v =
                (unsigned short)(((unsigned)(int)q0 & 0xFFu) | (((unsigned)(int)q1 & 0xFFu) << 8));
            *reinterpret_cast<unsigned short *>(qr + 32 * b + 2 * p) = v;
        }
    }
    if (tid == 0) x_scales[m] = amax > 0.0 ? (float)(amax / denom) : 0.f;
}

hipError_t launch_had32_quant(const uint16_t *X, const int8_t *signs, int64_t M, int64_t K,
                              int8_t *Xq, float *x_scales, double denom, hipStream_t s) {
    hipLaunchKernelGGL(had32_quant_kernel, dim3((unsigned)M), dim3(HQ_THREADS), 0, s, X, signs,
                       (int)K, Xq, x_scales, denom);
    return hipGetLastError();
}

}  // namespace qg
