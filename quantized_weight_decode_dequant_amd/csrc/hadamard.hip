// Block-diagonal randomized Hadamard-32 rotation followed by per-row int8
// quantization of the activations (Uzu page, fange-kb.cn, section "How Uzu
// optimizes bytes and tokens per pass": +-1 Hadamard entries and one global
// scale, random sign flips applied before the mixing, independent blocks of
// 32 chosen to match a 32-wide SIMD group, fully invertible; activations are
// quantized to 8 bits on the fly so verification runs on the int8 matrix
// path).
//
// One workgroup of 1024 threads per activation row.  Each 32-lane half of a
// wavefront owns one block of 32 at a time: lane i loads d_i * x_i and the
// five butterfly stages (xor 1, 2, 4, 8, 16) produce z_i = sum_j
// (-1)^popcount(i & j) d_j x_j (Sylvester order).  The sums are carried in
// fp64, where a signed sum of 32 bf16 values is exact, so the quantization
// decision below sees the exact z.  Pass 1 finds amax = max |z| over the row;
// pass 2 recomputes z (x is cache-resident by then) and writes
// round-half-even(z * 127 / amax), with the fp64 division correctly rounded.
#include "qg_internal.h"

namespace qg {

constexpr int HQ_THREADS = 1024;
constexpr int HQ_CHUNK = 4;  // blocks per half-wave per step (loads issued together)

__device__ __forceinline__ double fwht32(double v, int l32) {
#pragma unroll
    for (int s = 1; s < 32; s <<= 1) {
        const double o = __shfl_xor(v, s);
        v = (l32 & s) ? (o - v) : (v + o);
    }
    return v;
}

__global__ void __launch_bounds__(HQ_THREADS)
had32_quant_kernel(const uint16_t *__restrict__ X, const int8_t *__restrict__ signs, int K,
                   int8_t *__restrict__ Xq, float *__restrict__ x_scales, double denom) {
    __shared__ double wmax[HQ_THREADS / 64];
    const int m = blockIdx.x;
    const int tid = threadIdx.x, l32 = tid & 31, hw = tid >> 5;
    constexpr int HW = HQ_THREADS / 32;  // half-waves per workgroup
    const int nblk = K / 32;
    const uint16_t *xr = X + (size_t)m * K;
    double amax = 0.0;
    for (int b0 = hw; b0 < nblk; b0 += HW * HQ_CHUNK) {
        double v[HQ_CHUNK];
#pragma unroll
        for (int c = 0; c < HQ_CHUNK; ++c) {
            const int b = b0 + c * HW;
            const int k = 32 * b + l32;
            v[c] = (b < nblk) ? (double)signs[k] * (double)bf16_lo(xr[k]) : 0.0;
        }
#pragma unroll
        for (int c = 0; c < HQ_CHUNK; ++c) amax = fmax(amax, fabs(fwht32(v[c], l32)));
    }
    // row maximum: wave, then across waves
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) amax = fmax(amax, __shfl_xor(amax, s));
    if ((tid & 63) == 0) wmax[tid >> 6] = amax;
    __syncthreads();
    amax = 0.0;
#pragma unroll
    for (int w = 0; w < HQ_THREADS / 64; ++w) amax = fmax(amax, wmax[w]);

    int8_t *qr = Xq + (size_t)m * K;
    for (int b0 = hw; b0 < nblk; b0 += HW * HQ_CHUNK) {
        double v[HQ_CHUNK];
#pragma unroll
        for (int c = 0; c < HQ_CHUNK; ++c) {
            const int b = b0 + c * HW;
            const int k = 32 * b + l32;
            v[c] = (b < nblk) ? (double)signs[k] * (double)bf16_lo(xr[k]) : 0.0;
        }
#pragma unroll
        for (int c = 0; c < HQ_CHUNK; ++c) {
            const double z = fwht32(v[c], l32);
            const int b = b0 + c * HW;
            if (b < nblk) {
                double q = 0.0;
                if (amax > 0.0) {
                    q = rint(z * 127.0 / amax);
                    q = fmin(fmax(q, -127.0), 127.0);
                }
                qr[32 * b + l32] = (int8_t)(int)q;
            }
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
