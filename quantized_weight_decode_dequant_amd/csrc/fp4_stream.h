// Device helpers shared by the MXFP4 kernels: a batch of 4 tiles of one
// rowblock held in registers, and its loads through a buffer resource.
// Tile layout (2176 B, 16 rows x 256 k): lane l holds 16 bytes of codes of
// each half j (k = 128j + 32(l >> 4) .. +32 of row l & 15) and one E8M0 byte
// per half at 2048 + 64j + l.
#pragma once

#include "qg_internal.h"

namespace qg {

constexpr int MS_TPB = 4;  // tiles per batch

struct Fp4Batch {
    u32x4_t c0[MS_TPB], c1[MS_TPB];
    unsigned e0[MS_TPB], e1[MS_TPB];
};

__device__ __forceinline__ unsigned buf_ld_u8(__amdgpu_buffer_rsrc_t r, unsigned voff,
                                              unsigned soff) {
    return (unsigned)__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 2);
}

// One tile's loads into slot j of B (tile tp of the buffer, clamped to its
// last of pn tiles).
__device__ __forceinline__ void fp4_tile_load(Fp4Batch &B, int j, __amdgpu_buffer_rsrc_t rs,
                                              int tp, int pn, int lane) {
    const unsigned to = (unsigned)min(tp, pn - 1) * FP4_TILE_BYTES;
    B.c0[j] = buf_ld_x4(rs, 16u * lane, to);
    B.c1[j] = buf_ld_x4(rs, 1024u + 16u * lane, to);
    B.e0[j] = buf_ld_u8(rs, 2048u + lane, to);
    B.e1[j] = buf_ld_u8(rs, 2112u + lane, to);
}

}  // namespace qg
