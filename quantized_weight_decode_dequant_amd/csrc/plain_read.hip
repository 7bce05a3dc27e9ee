// Plain streaming read of a device buffer: the practical ceiling of every
// HBM-bound kernel in this library, measured on the same GPU in the same run
// ("MLX Runner: An Inference Engine You Can Read", section "Optimized against
// a known ceiling", and the Uzu page, section "Why batch-one decoding is
// memory-bound", both rate a decode against bandwidth divided by bytes).
//
// Workgroup j (8 waves) reads the contiguous 16-byte slots [j*n/G,
// (j+1)*n/G) with non-temporal 16-byte loads, 8 slots in flight per lane
// (each wave step covers 8 consecutive 1 KB slabs, a workgroup step 64 KB),
// XORs every word it read and writes the result to sink[j], so no load can be
// dropped.  On MI355X this layout (a contiguous chunk per workgroup,
// non-temporal) read fastest of the grid-stride and regular-load variants
// tried, and 8-wave workgroups 1-2% faster than 4- or 12-wave ones (4 GiB:
// 7.13-7.26 TB/s against 6.99-7.14; 4 or 16 slots in flight per lane, or
// loads without the non-temporal hint, are slower).
#include "qg_internal.h"

namespace qg {

constexpr int PR_U = 8;
constexpr int PR_THREADS = 512;

__global__ void __launch_bounds__(PR_THREADS)
plain_read_kernel(const u32x4_t *__restrict__ p, size_t n16, uint32_t *__restrict__ sink) {
    const size_t G = gridDim.x, j = blockIdx.x;
    const size_t b0 = j * n16 / G, b1 = (j + 1) * n16 / G;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr size_t SLAB = (size_t)PR_THREADS * PR_U;  // slots per workgroup step
    const size_t nfull = (b1 - b0) / SLAB;
    unsigned acc = 0;
    const u32x4_t *q = p + b0 + (size_t)wave * 64 * PR_U + lane;
    for (size_t t = 0; t < nfull; ++t, q += SLAB) {
        u32x4_t v[PR_U];
#pragma unroll
        for (int u = 0; u < PR_U; ++u)
            v[u] = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4_t *)(q + u * 64));
#pragma unroll
        for (int u = 0; u < PR_U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // the rest of the chunk, one slot per thread at a time
    for (size_t k = b0 + nfull * SLAB + threadIdx.x; k < b1; k += PR_THREADS) {
        const u32x4_t v = p[k];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // XOR over the workgroup: shuffles within the wave, then LDS
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    __shared__ unsigned part[PR_THREADS / 64];
    if (lane == 0) part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned t = 0;
#pragma unroll
        for (int w = 0; w < PR_THREADS / 64; ++w) t ^= part[w];
        st_global<uint32_t>(sink, j, t);
    }
}

hipError_t launch_plain_read(const void *buf, size_t bytes, uint32_t *sink, int grid,
                             hipStream_t s) {
    hipLaunchKernelGGL(plain_read_kernel, dim3(grid), dim3(PR_THREADS), 0, s,
                       reinterpret_cast<const u32x4_t *>(buf), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace qg
