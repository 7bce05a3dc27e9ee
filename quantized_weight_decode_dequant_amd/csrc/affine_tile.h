// Device helpers of the affine weight family shared by its GEMV and skinny
// kernels: the bit-plane layout of a tile (see qg_internal.h), a lane's words
// of one tile, and their unpacking into bf16 pairs 128 + q.
#pragma once

#include "qg_internal.h"

namespace qg {

// ------------------------------------------------------------ plane layout
template <int BITS>
struct AffPlanes;
template <> struct AffPlanes<2> { static constexpr int NP = 1, W0 = 2, W1 = 0, O1 = 0; };
template <> struct AffPlanes<3> { static constexpr int NP = 2, W0 = 2, W1 = 1, O1 = 2; };
template <> struct AffPlanes<4> { static constexpr int NP = 1, W0 = 4, W1 = 0, O1 = 0; };
template <> struct AffPlanes<5> { static constexpr int NP = 2, W0 = 4, W1 = 1, O1 = 4; };
template <> struct AffPlanes<6> { static constexpr int NP = 2, W0 = 4, W1 = 2, O1 = 4; };
template <> struct AffPlanes<8> { static constexpr int NP = 2, W0 = 4, W1 = 4, O1 = 4; };

// 3-bit codes: the bit position, within each 16-bit half of the tile's
// plane-1 word, of bit 2 of pair j's codes (j = 0..15).  Pair j's plane-0
// field is read from a copy of its plane-0 word shifted by 0, 6 or 12, at
// bits 2r..2r+1 with r = (j % 8) % 3, and its plane-1 bit belongs at bit
// 2r + 2.  The positions are chosen so that pairs of different r share the
// shift that brings their bits there (j = 0-2 by -2, 3-5 by -1, 8-10 by 4,
// 11-13 by 5, 6-7 by 10, 14-15 by 11): six shifts of the plane-1 word serve
// the 16 pairs.
__host__ __device__ constexpr int ag3_pos(int j) {
    return j < 6    ? 2 * (j % 3) + j / 3
           : j < 8  ? 12 + 2 * (j - 6)
           : j < 14 ? 6 + 2 * ((j - 8) % 3) + (j - 8) / 3
                    : 13 + 2 * (j - 14);
}

__device__ __forceinline__ unsigned buf_ld_x1(__amdgpu_buffer_rsrc_t r, unsigned voff,
                                              unsigned soff) {
    return (unsigned)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 2);
}

template <int W>
__device__ __forceinline__ void ag_ld(unsigned (&d)[W], __amdgpu_buffer_rsrc_t r, unsigned voff,
                                      unsigned soff) {
    if constexpr (W == 4) {
        const u32x4_t v = buf_ld_x4(r, voff, soff);
        d[0] = v[0], d[1] = v[1], d[2] = v[2], d[3] = v[3];
    } else if constexpr (W == 2) {
        const u32x2_t v = buf_ld_x2(r, voff, soff);
        d[0] = v[0], d[1] = v[1];
    } else {
        d[0] = buf_ld_x1(r, voff, soff);
    }
}

// One tile's words for this lane: the plane words and the (scale, bias)
// words of its row's GPT groups.
template <int BITS, int GPT>
struct AgTile {
    typedef AffPlanes<BITS> PL;
    unsigned p0[PL::W0];
    unsigned p1[PL::NP == 2 ? PL::W1 : 1];
    unsigned sb[GPT];
};

// Tile tp (clamped to the last of pn) of the buffer rs (tiles of tb bytes).
template <int BITS, int GPT>
__device__ __forceinline__ void ag_tile_load(AgTile<BITS, GPT> &T, __amdgpu_buffer_rsrc_t rs,
                                             int tp, int pn, unsigned tb, int lane) {
    typedef AffPlanes<BITS> PL;
    const unsigned to = (unsigned)min(tp, pn - 1) * tb;
    ag_ld<PL::W0>(T.p0, rs, 4u * PL::W0 * lane, to);
    if constexpr (PL::NP == 2) ag_ld<PL::W1>(T.p1, rs, 256u * PL::W0 + 4u * PL::W1 * lane, to);
    ag_ld<GPT>(T.sb, rs, 256u * BITS + 4u * GPT * (lane & 15), to);
}

constexpr unsigned AG_MAGIC = 0x43004300u;  // bf16 128 in both halves

// The constants of the unpack, held in VGPRs: gfx9 VOP3 instructions read at
// most one SGPR or literal, so with the mask and the magic both in registers
// (v & mask) | magic selects to one v_and_or_b32.  Made opaque once per
// kernel so that the compiler does not re-materialize them as literals at
// every use.  m0 masks a code of plane 0 in both halves; m1 a code of plane
// 1 moved to its place above plane 0 (8 bits: the high nibble in place).
struct AgConsts {
    unsigned magic, m0, m1;
};

__device__ __forceinline__ unsigned ag_opaque(unsigned c) {
    asm volatile("" : "+v"(c));
    return c;
}

template <int BITS>
__device__ __forceinline__ AgConsts ag_consts() {
    typedef AffPlanes<BITS> PL;
    constexpr unsigned m0 = ((1u << PL::W0) - 1u) * 0x00010001u;
    constexpr unsigned m1 =
        BITS == 8 ? 0x000F000Fu : ((((1u << PL::W1) - 1u) << PL::O1) * 0x00010001u);
    return AgConsts{ag_opaque(AG_MAGIC), ag_opaque(m0), PL::NP == 2 ? ag_opaque(m1) : 0u};
}

// (a & m) | c, kept whole: the result passes through an empty asm statement
// (no instruction), so the compiler cannot regroup it with the and-or it
// feeds (two and-ors would become two ands and an or3).  No instruction of
// these kernels is written in asm: the compiler does not count an asm
// instruction in its hazard checks, and an asm VALU write next to an MFMA
// (to a VGPR the MFMA reads within 2 wait states, or to one it has yet to
// write) corrupts the product.
__device__ __forceinline__ unsigned ag_and_or(unsigned a, unsigned m, unsigned c) {
    unsigned r = (a & m) | c;
    asm("" : "+v"(r));
    return r;
}

// Pair j (0..15; a compile-time index once unrolled) as two bf16 values
// 128 + q, one per 16-bit half (for 8 bits: 128 + the low nibble; the high
// nibble's pair comes from ag_pair_hi).  Plane 1's bits are shifted straight
// to their place above plane 0's and merged in by a second and-or.
template <int BITS, int GPT>
__device__ __forceinline__ unsigned ag_bf16_pair(const AgTile<BITS, GPT> &T, int j,
                                                 const AgConsts &k) {
    typedef AffPlanes<BITS> PL;
    constexpr int PER0 = 16 / PL::W0;
    const unsigned a = T.p0[j / PER0] >> (PL::W0 * (j % PER0));
    if constexpr (PL::NP == 2 && BITS != 8) {
        constexpr int PER1 = 16 / PL::W1;
        const int sh = (BITS == 3 ? ag3_pos(j) : PL::W1 * (j % PER1)) - PL::O1;
        const unsigned w = T.p1[j / PER1];
        return ((sh >= 0 ? w >> sh : w << -sh) & k.m1) | ag_and_or(a, k.m0, k.magic);
    } else {
        return (a & k.m0) | k.magic;
    }
}
template <int BITS, int GPT>
__device__ __forceinline__ unsigned ag_pair_hi(const AgTile<BITS, GPT> &T, int j,
                                               const AgConsts &k) {
    return ((T.p1[j / 4] >> (4 * (j % 4))) & k.m1) | k.magic;
}

__device__ __forceinline__ float ag_scale(unsigned sb, bool bf16) {
    return bf16 ? bf16_lo(sb) : f16_lo(sb);
}
__device__ __forceinline__ float ag_bias(unsigned sb, bool bf16) {
    return bf16 ? bf16_hi(sb) : f16_hi(sb);
}

}  // namespace qg
