// Canonical -> packed weight layouts (see qg_internal.h for the layouts).
// Weights are packed once at load time and never stored dequantized
// ("MLX Runner: An Inference Engine You Can Read", section "Architecture: one
// command buffer per token": one aligned copy of the weights, multiplied
// against the packed codes directly).  Each thread writes one 16-byte slot of
// the packed buffer, so the writes are fully coalesced.
#include "qg_internal.h"

namespace qg {

size_t q4_packed_bytes(int64_t N, int64_t K) {
    return (size_t)ceil_div(N, RB) * (size_t)ceil_div(K, Q4_TILE_K) * Q4_TILE_BYTES;
}
size_t q8_packed_bytes(int64_t N, int64_t K) {
    return (size_t)ceil_div(N, RB) * (size_t)ceil_div(K, Q8_TILE_K) * Q8_TILE_BYTES;
}
size_t fp4_packed_bytes(int64_t N, int64_t K) {
    return (size_t)ceil_div(N, RB) * (size_t)ceil_div(K, FP4_TILE_K) * FP4_TILE_BYTES;
}

size_t q8row_packed_bytes(int64_t N, int64_t K) {
    return (size_t)ceil_div(N, RB) *
           ((size_t)ceil_div(K, Q8R_TILE_K) * Q8R_TILE_BYTES + Q8R_RB_TAIL);
}

// Canonical word: element i (0..7) in bits 4i.  Packed word: element 2j in
// bits 4j, element 2j+1 in bits 16+4j.
__device__ __forceinline__ unsigned q4_interleave(unsigned cw) {
    unsigned out = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        unsigned nib = (cw >> (4 * i)) & 0xFu;
        int pos = (i & 1) ? 16 + 4 * (i >> 1) : 4 * (i >> 1);
        out |= nib << pos;
    }
    return out;
}

__global__ void __launch_bounds__(256)
pack_q4_kernel(const uint32_t *__restrict__ codes, const uint16_t *__restrict__ scales,
               const uint16_t *__restrict__ biases, int64_t N, int64_t K, int64_t P,
               int64_t nslots, uint4 *__restrict__ out) {
    const int64_t slot_id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (slot_id >= nslots) return;
    const int64_t tile = slot_id / 72;
    const int slot = (int)(slot_id % 72);
    const int64_t rb = tile / P, p = tile % P;
    const int64_t G = K / 64, KW = K / 8;
    uint4 v;
    if (slot < 64) {
        const int l = slot;
        const int64_t n = rb * RB + (l & 15);
        const int kg = l >> 4;
        unsigned w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = j >> 1, h = j & 1;
            const int64_t e0 = p * 128 + 64 * t + 32 * h + 8 * kg;
            w[j] = (n < N && e0 < K) ? q4_interleave(codes[n * KW + e0 / 8]) : 0u;
        }
        v = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
        unsigned w[4];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int64_t n = rb * RB + 2 * (slot - 64) + rr;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int64_t g = 2 * p + t;
                unsigned sb = 0;
                if (n < N && g < G)
                    sb = (unsigned)scales[n * G + g] | ((unsigned)biases[n * G + g] << 16);
                w[2 * rr + t] = sb;
            }
        }
        v = make_uint4(w[0], w[1], w[2], w[3]);
    }
    out[slot_id] = v;
}

__global__ void __launch_bounds__(256)
pack_q8_kernel(const int8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
               int64_t N, int64_t K, int64_t P, int64_t nslots, uint4 *__restrict__ out) {
    const int64_t slot_id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (slot_id >= nslots) return;
    const int64_t tile = slot_id / 136;
    const int slot = (int)(slot_id % 136);
    const int64_t rb = tile / P, p = tile % P;
    const int64_t G = K / 32;
    unsigned w[4] = {0u, 0u, 0u, 0u};
    if (slot < 128) {
        const int j = slot >> 6, l = slot & 63;
        const int64_t n = rb * RB + (l & 15);
        const int kg = l >> 4;
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
            const int64_t k0 = p * 128 + 32 * (2 * j + gg) + 8 * kg;
            if (n < N && k0 < K) {
                const uint2 c = *reinterpret_cast<const uint2 *>(codes + n * K + k0);
                w[2 * gg] = c.x;
                w[2 * gg + 1] = c.y;
            }
        }
    } else {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int64_t n = rb * RB + 2 * (slot - 128) + rr;
#pragma unroll
            for (int gp = 0; gp < 2; ++gp) {
                unsigned lo = 0, hi = 0;
                const int64_t g0 = 4 * p + 2 * gp;
                if (n < N && g0 < G) lo = scales[n * G + g0];
                if (n < N && g0 + 1 < G) hi = scales[n * G + g0 + 1];
                w[2 * rr + gp] = lo | (hi << 16);
            }
        }
    }
    out[slot_id] = make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ void __launch_bounds__(256)
pack_fp4_kernel(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                int64_t N, int64_t K, int64_t P, int64_t nslots, uint4 *__restrict__ out) {
    const int64_t slot_id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (slot_id >= nslots) return;
    const int64_t tile = slot_id / 136;
    const int slot = (int)(slot_id % 136);
    const int64_t rb = tile / P, p = tile % P;
    const int64_t NB = K / 32;  // scale blocks per row
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (slot < 128) {
        const int j = slot >> 6, l = slot & 63;
        const int64_t n = rb * RB + (l & 15);
        const int64_t blk = 8 * p + 4 * j + (l >> 4);
        if (n < N && blk < NB)
            v = *reinterpret_cast<const uint4 *>(codes + n * (K / 2) + blk * 16);
    } else {
        unsigned w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int b = (slot - 128) * 16 + i;
            const int j = b >> 6, l = b & 63;
            const int64_t n = rb * RB + (l & 15);
            const int64_t blk = 8 * p + 4 * j + (l >> 4);
            unsigned e = (n < N && blk < NB) ? scales[n * NB + blk] : 0u;
            w[i >> 2] |= e << (8 * (i & 3));
        }
        v = make_uint4(w[0], w[1], w[2], w[3]);
    }
    out[slot_id] = v;
}

static inline unsigned grid_for(int64_t n, int block) { return (unsigned)ceil_div(n, block); }

// Per-row int8: a rowblock is P tiles of 128 slots, then 4 slots of row
// scales.  Codes are copied in k order (16 bytes = 16 consecutive k).
__global__ void __launch_bounds__(256)
pack_q8row_kernel(const int8_t *__restrict__ codes, const float *__restrict__ scales, int64_t N,
                  int64_t K, int64_t P, int64_t nslots, uint4 *__restrict__ out) {
    const int64_t slot_id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (slot_id >= nslots) return;
    const int64_t per_rb = P * 128 + Q8R_RB_TAIL / 16;
    const int64_t rb = slot_id / per_rb;
    const int64_t s = slot_id - rb * per_rb;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (s < P * 128) {
        const int64_t p = s / 128;
        const int t = (int)(s % 128), j = t >> 6, l = t & 63;
        const int64_t n = rb * RB + (l & 15);
        const int64_t k0 = p * Q8R_TILE_K + 64 * j + 16 * (l >> 4);
        if (n < N && k0 < K) v = *reinterpret_cast<const uint4 *>(codes + n * K + k0);
    } else {
        const int q = (int)(s - P * 128);
        unsigned w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t n = rb * RB + 4 * q + r;
            w[r] = n < N ? __float_as_uint(scales[n]) : 0u;
        }
        v = make_uint4(w[0], w[1], w[2], w[3]);
    }
    out[slot_id] = v;
}

hipError_t launch_pack_q8row(const int8_t *codes, const float *scales, int64_t N, int64_t K,
                             uint8_t *packed, hipStream_t s) {
    const int64_t P = ceil_div(K, Q8R_TILE_K);
    const int64_t nslots = ceil_div(N, RB) * (P * 128 + Q8R_RB_TAIL / 16);
    hipLaunchKernelGGL(pack_q8row_kernel, dim3(grid_for(nslots, 256)), dim3(256), 0, s, codes,
                       scales, N, K, P, nslots, reinterpret_cast<uint4 *>(packed));
    return hipGetLastError();
}

hipError_t launch_pack_q4(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                          int64_t N, int64_t K, uint8_t *packed, hipStream_t s) {
    const int64_t P = ceil_div(K, Q4_TILE_K);
    const int64_t nslots = ceil_div(N, RB) * P * (Q4_TILE_BYTES / 16);
    hipLaunchKernelGGL(pack_q4_kernel, dim3(grid_for(nslots, 256)), dim3(256), 0, s, codes,
                       scales, biases, N, K, P, nslots, reinterpret_cast<uint4 *>(packed));
    return hipGetLastError();
}

hipError_t launch_pack_q8(const int8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                          uint8_t *packed, hipStream_t s) {
    const int64_t P = ceil_div(K, Q8_TILE_K);
    const int64_t nslots = ceil_div(N, RB) * P * (Q8_TILE_BYTES / 16);
    hipLaunchKernelGGL(pack_q8_kernel, dim3(grid_for(nslots, 256)), dim3(256), 0, s, codes,
                       scales, N, K, P, nslots, reinterpret_cast<uint4 *>(packed));
    return hipGetLastError();
}

hipError_t launch_pack_fp4(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                           uint8_t *packed, hipStream_t s) {
    const int64_t P = ceil_div(K, FP4_TILE_K);
    const int64_t nslots = ceil_div(N, RB) * P * (FP4_TILE_BYTES / 16);
    hipLaunchKernelGGL(pack_fp4_kernel, dim3(grid_for(nslots, 256)), dim3(256), 0, s, codes,
                       scales, N, K, P, nslots, reinterpret_cast<uint4 *>(packed));
    return hipGetLastError();
}

}  // namespace qg

namespace qg {

// Device upload through kernel arguments: the words travel inside the kernel
// argument block, so the host buffer need not outlive the call and no
// host-side synchronization is needed.
constexpr int WW_WORDS = 896;
struct WordChunk {
    uint32_t n;
    uint32_t w[WW_WORDS];
};

__global__ void __launch_bounds__(256) write_words_kernel(WordChunk chunk, uint32_t *__restrict__ dst) {
    for (uint32_t i = threadIdx.x; i < chunk.n; i += blockDim.x) dst[i] = chunk.w[i];
}

hipError_t launch_write_words(const uint32_t *src, size_t nwords, uint32_t *dst, hipStream_t s) {
    for (size_t off = 0; off < nwords; off += WW_WORDS) {
        WordChunk c;
        c.n = (uint32_t)((nwords - off) < (size_t)WW_WORDS ? (nwords - off) : (size_t)WW_WORDS);
        for (uint32_t i = 0; i < c.n; ++i) c.w[i] = src[off + i];
        hipLaunchKernelGGL(write_words_kernel, dim3(1), dim3(256), 0, s, c, dst + off);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qg
