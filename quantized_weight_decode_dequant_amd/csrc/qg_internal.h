// Internal declarations shared by the HIP sources of the qgemv library.
// gfx950 (CDNA4) only: 64-lane wavefronts, MFMA matrix cores, 160 KB LDS/CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace qg {

// ---------------------------------------------------------------- packed layout
//
// Every packed format is a sequence of "tiles".  A tile covers 16 consecutive
// output rows (a rowblock) and a run of consecutive k; tiles are stored
// rowblock-major, so one rowblock's tiles are contiguous.  Inside a tile the
// first 1 KB (or 2 KB) holds the codes in the order a 64-lane wavefront reads
// them with one 128-bit load per lane: lane l serves row n = 16*rb + (l & 15)
// and k-slice kg = l >> 4.  This is also the operand layout of the
// 16x16x32 MFMA instructions (lane l holds 8 consecutive k of column l & 15,
// k-slice l >> 4), so one packed buffer feeds both the M = 1 VALU kernels and
// the M <= 32 MFMA kernels.  The scales follow the codes inside the tile.
//
// Q4 asymmetric group-64, tile = 128 k (2 groups), 1152 B:
//   [0, 1024)     lane l: 4 words; word 2t+h = group t of the tile, elements
//                 32h + 8kg .. +8.  Within a word element 2j sits in bits
//                 [4j, 4j+4) and element 2j+1 in bits [16+4j, 20+4j), so
//                 (w >> 4j) & 0x000F000F yields the pair (2j, 2j+1) as the
//                 two 16-bit halves of a register.
//   [1024, 1152)  16 rows x 2 groups x {fp16 scale, fp16 bias}: row r at
//                 1024 + 8r: (s0, b0, s1, b1).
// Q8 symmetric group-32, tile = 128 k (4 groups), 2176 B:
//   [0, 2048)     half j (1 KB each): lane l: 16 bytes = groups 2j, 2j+1 of
//                 the tile, 8 consecutive int8 each (k = 32g + 8kg .. +8).
//   [2048, 2176)  16 rows x 4 groups fp16 scales: row r at 2048 + 8r.
// MXFP4 group-32, tile = 256 k (8 blocks), 2176 B:
//   [0, 2048)     half j (1 KB each): lane l: 16 bytes = 32 E2M1 codes of
//                 block 4j + kg (k = 128j + 32kg .. +32), element 2i in the
//                 low nibble of byte i.
//   [2048, 2176)  E8M0 scale bytes: half j at 2048 + 64j + l.
// Q8_ROW (int8, one fp32 scale per row), tile = 128 k, 2048 B:
//   [0, 2048)     half j (1 KB each): lane l: 16 int8 codes of row l & 15,
//                 k = 64j + 16(l >> 4) .. +16, in k order.
//   A rowblock is its tiles followed by 64 B: the fp32 scales of its 16 rows.
// AFFINE (b-bit unsigned codes, group g, (scale, bias) fp16 or bf16), tile =
// 128 k, 256 b + 16 (128 / g) 4 bytes:
//   the codes as bit-planes of width 1, 2 or 4 (b = 2: {2}; 3: {2, 1};
//   4: {4}; 5: {4, 1}; 6: {4, 2}; 8: {4, 4}; plane p holds bits
//   [o_p, o_p + w_p) of each code).  Plane p occupies 256 w_p bytes; lane l
//   holds w_p words at 4 w_p l for 32 codes c_0..c_31 of row l & 15 in four
//   runs of 8: c_{8i+t} is k = 32i + 8(l >> 4) + t (so run i of all 64 lanes
//   covers k = 32i .. 32i + 32, one 32-k block: the k of one 16x16x32 MFMA
//   step, inside one group).  Pair j (codes 2j, 2j+1) sits in word
//   j / (16 / w_p), at bit w_p (j % (16 / w_p)) (code 2j) and 16 + the same
//   (code 2j+1), so a shift and an and-or yield both as the two halves; the
//   one exception is the 1-bit plane of 3-bit codes, where pair j's bits sit
//   at ag3_pos(j) and 16 + ag3_pos(j) (affine_tile.h), an order that lets
//   one shift serve three pairs.
//   [256 b, ...)  per (row r, group t of the tile): (scale | bias << 16) at
//   256 b + 4 (r (128 / g) + t).
// Rows past N and k past K are zero-filled (zero codes and zero scales).

constexpr int RB = 16;              // rows per rowblock
constexpr int Q4_TILE_K = 128;
constexpr int Q4_TILE_BYTES = 1152;
constexpr int Q8_TILE_K = 128;
constexpr int Q8_TILE_BYTES = 2176;
constexpr int FP4_TILE_K = 256;
constexpr int FP4_TILE_BYTES = 2176;
constexpr int Q8R_TILE_K = 128;
constexpr int Q8R_TILE_BYTES = 2048;
constexpr int Q8R_RB_TAIL = 64;  // the row scales after a rowblock's tiles
constexpr int AFF_TILE_K = 128;

// Affine-family format codes (QG_FMT_AFFINE in qgemv.h).
struct AffineFmt {
    int bits, group, bf16;  // bits 0 = not an affine code
};
inline AffineFmt affine_decode(int fmt) {
    AffineFmt f{0, 0, 0};
    if ((fmt & ~0xFF) != 0x100) return f;
    const int bits = (fmt >> 4) & 0xF, gc = (fmt >> 2) & 3;
    if (!(bits == 2 || bits == 3 || bits == 4 || bits == 5 || bits == 6 || bits == 8) || gc == 3)
        return f;
    f.bits = bits;
    f.group = 32 << gc;
    f.bf16 = fmt & 1;
    return f;
}
__host__ __device__ inline size_t affine_tile_bytes(int bits, int group) {
    return (size_t)256 * bits + (size_t)16 * (AFF_TILE_K / group) * 4;
}

// T-position MoE: (position, slot) pairs per call, and the most pairs of
// one expert that share one read of its weights.
constexpr int MOE_PAIRS_MAX = 2048;
constexpr int MOE_GROUP_ROWS_MAX = 4;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- work lists
// One entry per matrix of a grouped launch (device-resident, written by
// qg_batch_plan_build), or passed by value for a single-matrix launch.
// `units` is the number of scheduling units of the matrix: its rowblocks.
struct alignas(16) WorkItem {
    const uint8_t *packed;
    const void *x;   // bf16 [M][K]
    void *y;         // [M][N]
    int32_t N, K;
    int32_t P;       // 128-k tiles per row
    int32_t units;
    int32_t out_f32;
    int32_t pad;
};
static_assert(sizeof(WorkItem) == 48, "work item layout");

// First unit of each workgroup, in (item, unit) order; entry [grid] is the
// end sentinel.  Workgroup j processes [starts[j], starts[j+1]).
struct WorkStart {
    int32_t item, unit;
};

constexpr int WL_HEADER_BYTES = 64;
constexpr int WL_GRID_MAX = 4096;
constexpr uint32_t WL_MAGIC = 0x4C57'4751u;  // "QGWL"

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Arguments are validated by
// the C ABI layer before these are called.
hipError_t launch_pack_q4(const uint32_t *codes, const uint16_t *scales,
                          const uint16_t *biases, int64_t N, int64_t K,
                          uint8_t *packed, hipStream_t s);
hipError_t launch_pack_q8(const int8_t *codes, const uint16_t *scales,
                          int64_t N, int64_t K, uint8_t *packed, hipStream_t s);
hipError_t launch_pack_fp4(const uint8_t *codes, const uint8_t *scales,
                           int64_t N, int64_t K, uint8_t *packed, hipStream_t s);

// Q4 GEMV on the VALU for 1..q4_gemv_rows_max() activation rows (x is
// bf16 [M][K], y [M][N]); single matrix or a device work list
hipError_t launch_q4_gemv(const uint8_t *packed, const uint16_t *x, void *y, int64_t M,
                          int64_t N, int64_t K, bool out_f32, int cus, hipStream_t s);
size_t q4_gemv_lds_bytes(int64_t M);
int q4_gemv_wgs_per_cu(int64_t M);       // single matrices
int q4_gemv_list_wgs_per_cu(int64_t M);  // the work list
int q4_gemv_rows_max();
hipError_t launch_q4_gemv_list(const WorkItem *items, const WorkStart *starts,
                               int grid, int64_t M, hipStream_t s);
// streaming skinny kernel (one workgroup of 16 waves for M <= 16, 12 waves
// for M <= 32, per CU; the X slice of a segment staged whole in LDS)
int q4_skinny_stream_wgs_per_cu();
bool q4_skinny_stream_fits(int64_t N, int cus);
hipError_t launch_q4_skinny_stream(const uint8_t *packed, const uint16_t *X, void *Y,
                                   int64_t M, int64_t N, int64_t K, bool out_f32,
                                   int cus, hipStream_t s);
hipError_t launch_q4_skinny_stream_list(const WorkItem *items, const WorkStart *starts,
                                        int grid, int64_t M, hipStream_t s);
hipError_t launch_plain_read(const void *buf, size_t bytes, uint32_t *sink, int grid,
                             hipStream_t s);
hipError_t launch_write_words(const uint32_t *src, size_t nwords, uint32_t *dst,
                              hipStream_t s);
hipError_t launch_fp4_gemv(const uint8_t *packed, const uint16_t *x, void *y,
                           int64_t N, int64_t K, bool out_f32, int cus,
                           hipStream_t s);
hipError_t launch_q4_skinny(const uint8_t *packed, const uint16_t *X, void *Y,
                            int64_t M, int64_t N, int64_t K, bool out_f32,
                            int cus, hipStream_t s);
hipError_t launch_q8_skinny(const uint8_t *packed, const int8_t *X,
                            const float *x_scales, void *Y, int64_t M,
                            int64_t N, int64_t K, int out_mode, int cus,
                            hipStream_t s);
hipError_t launch_had32_quant(const uint16_t *X, const int8_t *signs,
                              int64_t M, int64_t K, int8_t *Xq,
                              float *x_scales, double denom,
                              hipStream_t s);
// The single-token MoE layer; h, the per-slot partials and (unless
// status_out is given) the status word live in `workspace`.
hipError_t launch_moe(const uint8_t *pg, const uint8_t *pu, const uint8_t *pd,
                      int64_t E, int64_t H, int64_t F, const uint16_t *x,
                      int top_k, const int32_t *ids, const float *w,
                      uint8_t *workspace, void *y, bool out_f32, int cus,
                      hipStream_t s, unsigned *status_out = nullptr);

hipError_t launch_moe_combine(const float *part, const int32_t *ids, const float *w,
                              int64_t E, int64_t H, int top_k, int T, void *y,
                              bool out_f32, unsigned *status, hipStream_t s);
hipError_t launch_moe_skinny(const uint8_t *pg, const uint8_t *pu, const uint8_t *pd,
                             int64_t E, int64_t H, int64_t F, int T,
                             const uint16_t *X, int top_k, const int32_t *ids,
                             const float *w, uint8_t *workspace, void *Y,
                             bool out_f32, int cus, hipStream_t s);
// Positions whose x (or h) one group of the T-position MoE stages at once.
int moe_skinny_group_rows(int64_t H, int64_t F);

hipError_t launch_pack_q8row(const int8_t *codes, const float *scales, int64_t N,
                            int64_t K, uint8_t *packed, hipStream_t s);
hipError_t launch_q8row_gemv(const uint8_t *packed, const uint16_t *x, void *y,
                             int64_t N, int64_t K, bool out_f32, int cus,
                             hipStream_t s);
// the row-scale int8 GEMV over a device work list (kmax = the largest K)
hipError_t launch_q8row_gemv_list(const WorkItem *items, const WorkStart *starts, int grid,
                                  int64_t kmax, hipStream_t s);
int q8row_gemv_wgs_per_cu();
size_t q8row_packed_bytes(int64_t N, int64_t K);
size_t affine_packed_bytes(int bits, int group, int64_t N, int64_t K);
hipError_t launch_pack_affine(const uint8_t *codes, const uint16_t *scales,
                              const uint16_t *biases, int bits, int group,
                              int64_t N, int64_t K, uint8_t *packed,
                              hipStream_t s);
hipError_t launch_affine_gemv(const uint8_t *packed, const uint16_t *x, void *y,
                              int bits, int group, bool bf16_scales, int64_t N,
                              int64_t K, bool out_f32, int cus, hipStream_t s);
// the affine GEMV over a device work list (M = 1; every item of one format);
// kmax = the largest K of the list (sizes the LDS)
hipError_t launch_affine_gemv_list(const WorkItem *items, const WorkStart *starts, int grid,
                                   int64_t kmax, int bits, int group, bool bf16_scales,
                                   hipStream_t s);
int affine_gemv_wgs_per_cu();
hipError_t launch_affine_skinny(const uint8_t *packed, const uint16_t *X, void *Y,
                                int bits, int group, bool bf16_scales, int64_t M,
                                int64_t N, int64_t K, bool out_f32, int cus,
                                hipStream_t s);
// the affine skinny product over a device work list (M = 2..32; every item
// of one format), one workgroup per CU
hipError_t launch_affine_skinny_list(const WorkItem *items, const WorkStart *starts, int grid,
                                     int bits, int group, bool bf16_scales, int64_t M,
                                     hipStream_t s);
int affine_skinny_wgs_per_cu();

size_t q4_packed_bytes(int64_t N, int64_t K);
size_t q8_packed_bytes(int64_t N, int64_t K);
size_t fp4_packed_bytes(int64_t N, int64_t K);

}  // namespace qg

// ---------------------------------------------------------------- device helpers
#if defined(__HIPCC__)
namespace qg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    unsigned u = __builtin_bit_cast(unsigned, f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu))
        return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_lo(unsigned w) {
    return __builtin_bit_cast(float, w << 16);
}
__device__ __forceinline__ float bf16_hi(unsigned w) {
    return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

__device__ __forceinline__ float f16_lo(unsigned w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(unsigned w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// fp32 accumulate += (a.lo * b.lo + a.hi * b.hi) for bf16 pairs (single
// rounding; v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(unsigned a, unsigned b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

// E8M0 byte e -> the fp32 whose exponent field is e (2^(e-127) for
// 1 <= e <= 254); the gfx950 scaled FP4 converts use only the exponent of
// their fp32 scale operand.
__device__ __forceinline__ float e8m0_as_f32(unsigned e) {
    return __builtin_bit_cast(float, (e & 0xFFu) << 23);
}

// Two E2M1 codes of byte SEL of w, times the scale, as a bf16 pair (exact for
// the E8M0 range used here).
template <int SEL>
__device__ __forceinline__ unsigned fp4_pair_bf16(unsigned w, float scale) {
    return __builtin_bit_cast(
        unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL));
}
template <int SEL>
__device__ __forceinline__ f32x2_t fp4_pair_f32(unsigned w, float scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, SEL);
}

// MI355X dispatches the workgroups of a launch to its 8 XCDs in turn
// (workgroup b runs on XCD b mod 8), and each XCD has its own L2.  This maps
// the hardware index b to a work index so that consecutive work indices run
// on the same XCD: XCD x takes the x-th run of about grid / 8 consecutive
// indices.  Work split into contiguous ranges in index order (rowblocks of
// one matrix, one activation tile) then shares the L2 of one XCD instead of
// being spread over all eight.  A bijection of [0, grid) for every grid.
constexpr int XCDS = 8;
__device__ __forceinline__ int xcd_work_index(int b, int grid) {
    const int q = grid / XCDS, r = grid % XCDS;
    const int x = b % XCDS, i = b / XCDS;
    return x * q + min(x, r) + i;
}

// Streaming (non-temporal) load through the global address space.  Pointers
// read from memory (work lists) are otherwise generic, which makes the
// compiler emit FLAT loads; those also count against the LDS counter, so every
// LDS read would wait for the outstanding HBM loads.
template <typename T>
__device__ __forceinline__ T ld_nt(const T *p) {
    return __builtin_nontemporal_load((const __attribute__((address_space(1))) T *)p);
}

// A wave-uniform pointer made opaque to the optimizer (readfirstlane of both
// halves), so address arithmetic on it stays scalar instead of being folded
// into per-lane 64-bit vector offsets.
__device__ __forceinline__ const uint8_t *uniform_ptr(const uint8_t *p) {
    const unsigned long long v = reinterpret_cast<unsigned long long>(p);
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
    return reinterpret_cast<const uint8_t *>(((unsigned long long)hi << 32) | lo);
}

// Buffer resource over [base, base + bytes) for raw buffer loads (gfx9
// descriptor word 3).  Loads through it take the wave-uniform part of the
// address in an SGPR (soffset) and one 32-bit per-lane VGPR offset.  The
// range check applies to the VGPR offset: a load whose VGPR offset is at or
// past `bytes` reads zero without touching memory (so does every load through
// a resource of 0 bytes), but the SGPR offset is added unchecked, so callers
// keep SGPR offsets inside the buffer.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Non-temporal (streaming) buffer loads: aux = slc.
__device__ __forceinline__ u32x4_t buf_ld_x4(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2));
}
__device__ __forceinline__ u32x2_t buf_ld_x2(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 2));
}

template <typename T>
__device__ __forceinline__ T ld_global(const T *p) {
    return *(const __attribute__((address_space(1))) T *)p;
}

// Store through the global address space.  Output pointers read from a work
// list are generic, and a FLAT store also counts against the LDS counter, so
// every later LDS read of the wave would wait for the store to complete.
template <typename T>
__device__ __forceinline__ void st_global(void *base, size_t i, T v) {
    ((__attribute__((address_space(1))) T *)base)[i] = v;
}

// The same with the non-temporal hint: for whole-line runs of output written
// in the middle of a weight stream (measured: lighter on the read stream than
// plain stores; slower for 2-byte pieces).
template <typename T>
__device__ __forceinline__ void st_global_nt(void *base, size_t i, T v) {
    __builtin_nontemporal_store(v, ((__attribute__((address_space(1))) T *)base) + i);
}

// The two constants of the nibble unpack, held in VGPRs.  gfx9 VOP3
// instructions read at most one SGPR or literal, so with both operands in
// registers (a & mask) | magic selects to a single v_and_or_b32.  They are
// moved into VGPRs once and made opaque by an empty asm statement (no
// instruction), so the compiler does not re-materialize them as literals at
// every use.
struct Q4Consts {
    unsigned mask;   // 0x000F000F
    unsigned magic;  // bf16 128.0 twice
};

__device__ __forceinline__ Q4Consts q4_consts() {
    Q4Consts k{0x000F000Fu, 0x43004300u};
    asm volatile("" : "+v"(k.mask));
    asm volatile("" : "+v"(k.magic));
    return k;
}

// The four bf16 pairs (128 + q_2j, 128 + q_2j+1), j = 0..3, of a packed Q4 word.
__device__ __forceinline__ void q4_unpack(unsigned w, const Q4Consts &k, unsigned out[4]) {
    out[0] = (w & k.mask) | k.magic;
    out[1] = ((w >> 4) & k.mask) | k.magic;
    out[2] = ((w >> 8) & k.mask) | k.magic;
    out[3] = ((w >> 12) & k.mask) | k.magic;
}

// Eight 4-bit codes of a packed Q4 word as the bf16x8 MFMA operand
// (128 + q_0, ..., 128 + q_7).
__device__ __forceinline__ bf16x8_t q4_word_to_bf16x8(unsigned w, const Q4Consts &k) {
    unsigned o[4];
    q4_unpack(w, k, o);
    u32x4_t v = {o[0], o[1], o[2], o[3]};
    return __builtin_bit_cast(bf16x8_t, v);
}

}  // namespace qg
#endif
