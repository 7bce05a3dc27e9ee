/*
 * qgemv.h -- C ABI of the weight-quantized decode GEMV / skinny GEMM library
 * for AMD Instinct MI355X (gfx950).
 *
 * What it computes.  Batch-one LLM decode streams every weight once per token
 * with about one multiply-add per weight, so it is bound by memory bandwidth
 * (Uzu on Apple M5, fange-kb.cn, section "Why batch-one decoding is
 * memory-bound"; "MLX Runner: An Inference Engine You Can Read", section
 * "Optimized against a known ceiling").  This library provides that product,
 * y = W x, for weights kept in quantized form and dequantized in registers,
 * plus its skinny form Y = X W^T for M <= 32 activation rows, which is how a
 * draft of 16-32 speculative tokens is verified in one pass (Uzu page,
 * section "Producing several tokens from one model pass").
 *
 * Weight formats (each matrix is stored [N, K]: N output rows, K inputs):
 *  - QG_FMT_Q4_ASYM_G64: 4-bit unsigned codes, one fp16 scale and one fp16
 *    bias per group of 64 consecutive k; weight = scale * code + bias
 *    ("MLX Runner", section "Architecture: one command buffer per token";
 *    asymmetric 4-bit per the Uzu page, section "How Uzu optimizes bytes and
 *    tokens per pass").
 *  - QG_FMT_Q8_SYM_G32: int8 codes in [-127, 127], one fp16 scale per group of
 *    32, multiplied by int8 activations (Uzu page, same section: 8-bit
 *    symmetric checkpoints; activations quantized to 8 bits on the fly after a
 *    block-diagonal randomized Hadamard-32 rotation).
 *  - QG_FMT_MXFP4_G32: E2M1 codes with one E8M0 scale per 32 values (Deltafin
 *    / Kimi K3 page, aihot.virxact.com, sections "How it works" and the compute
 *    list: fused MXFP4 dequant + GEMV for the routed experts).
 *  - QG_FMT_AFFINE(bits, group, bf16_scales): the affine family of "MLX
 *    Runner" (section "Architecture: one command buffer per token": weights
 *    stored as codes with a scale and a bias per group; the audit section
 *    lists its widths): unsigned codes of 2, 3, 4, 5, 6 or 8 bits, groups of
 *    32, 64 or 128 consecutive k, one scale and one bias per group in fp16
 *    (bf16_scales = 0) or bf16 (1); weight = scale * code + bias.  Decode
 *    GEMV (qgemv_run) and skinny product (qgemm_skinny_run).
 *  - QG_FMT_Q8_ROW: int8 codes (the full range -128..127) with one fp32 scale
 *    per output row, weight = scale[n] * code, against bf16 activations:
 *    weight-only int8 as in the Deltafin page's resident int8 spine and packed
 *    int8 output head (sections on the spine and the recent changes: int8 to
 *    fp32 conversion fused with the row scaling).
 *
 * Canonical (unpacked) layouts accepted by qgemv_pack, all row-major device
 * buffers:
 *  - Q4:    codes uint32 [N][K/8] (element k in bits 4*(k%8).., low nibble
 *           first); scales, biases fp16 [N][K/64].
 *  - Q8:    codes int8 [N][K];  scales fp16 [N][K/32];  biases NULL.
 *  - MXFP4: codes uint8 [N][K/2] (element 2i in the low nibble of byte i);
 *           scales uint8 E8M0 [N][K/32];  biases NULL.  Supported scale
 *           bytes are 1..252 (2^-126 .. 2^125), the range in which every
 *           E2M1 value times the scale is finite in bf16 and fp32.  From 253
 *           on, +-6 times the scale overflows (to infinity, and a zero
 *           activation times it to NaN); bytes 0 and 255 (2^-127 and NaN in
 *           the OCP MX definition) are outside the range too: the kernels
 *           use the byte as the exponent field of an fp32 scale, so 0 acts
 *           as a scale of 0 and 255 as infinity.  Results for blocks with
 *           unsupported scales are unspecified (the scales live in device
 *           memory, so the call cannot reject them).
 *  - Q8_ROW: codes int8 [N][K];  scales fp32 [N];  biases NULL.
 *  - AFFINE: codes uint8 [N][K], one code per byte (< 2^bits); scales and
 *           biases fp16 or bf16 [N][K/group].
 * The packed layout is opaque: a buffer produced by qgemv_pack for a given
 * (fmt, rows, K) is consumed only by calls with the same (fmt, N, K).
 *
 * Conventions for every call:
 *  - Every buffer is caller-owned device memory.  The library allocates no
 *    memory, frees none and never synchronizes; it keeps only a per-device
 *    cache of the compute-unit count.
 *  - `stream` is a hipStream_t (NULL = the default stream).  A call validates
 *    its arguments on the host, enqueues its kernels on `stream` and returns.
 *  - Validation happens before any HIP call, so an invalid call returns its
 *    error without touching the device.  Device pointers marked "16-B" must be
 *    16-byte aligned; others need their element's natural alignment.
 *  - A dimension of 0 (N = 0, M = 0, top_k = 0) is a valid empty problem:
 *    nothing is enqueued (moe_expert_gemv_run with top_k = 0 still writes
 *    y = 0).
 *  - Calls are re-entrant; calls on different streams may run concurrently
 *    as long as they do not write the same buffers.
 *  - No C++ exception crosses this interface.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QG_OK = 0,
    QG_EINVAL = -1,       /* NULL where a pointer is required; unknown enum value */
    QG_ESHAPE = -2,       /* dimension out of range (K not a multiple of the
                             format's block, M outside 0..32, top_k > E, ...) */
    QG_EALIGN = -3,       /* a device pointer violates its alignment */
    QG_ESIZE = -4,        /* packed_bytes / workspace_bytes is not the size the
                             layout needs */
    QG_EUNSUPPORTED = -5, /* format x output x entry point combination not provided */
    QG_EHIP = -6,         /* the HIP runtime reported an error */
    QG_EINTERNAL = -7     /* unexpected internal failure */
} qg_status;

typedef enum {
    QG_FMT_Q4_ASYM_G64 = 1,
    QG_FMT_Q8_SYM_G32 = 2,
    QG_FMT_MXFP4_G32 = 3,
    QG_FMT_Q8_ROW = 4
} qg_format;

/* Format code of an affine-family member: bits in {2, 3, 4, 5, 6, 8}, group
 * in {32, 64, 128}, bf16_scales 0 (fp16 scales and biases) or 1 (bf16).  Any
 * other combination gives a code the calls reject with QG_EINVAL. */
#define QG_FMT_AFFINE(bits, group, bf16_scales)                              \
    (0x100 | (((bits) & 0xF) << 4) |                                        \
     (((group) == 32 ? 0 : (group) == 64 ? 1 : (group) == 128 ? 2 : 3) << 2) | \
     ((bf16_scales) ? 1 : 0))

typedef enum {
    QG_OUT_BF16 = 0,       /* bf16, round to nearest even */
    QG_OUT_F32 = 1,        /* fp32, the accumulator as computed */
    QG_OUT_I32_GROUPS = 2  /* Q8 only: exact int32 group partials [M][N][K/32] */
} qg_out;

/* Human-readable name of a status code (static string, never NULL). */
const char *qg_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int qg_version(void);

/*
 * qgemv_pack -- convert canonical device tensors into the packed device
 * layout that the run calls stream with 128-bit coalesced loads.  Weights are
 * packed once at load time and never stored dequantized ("MLX Runner",
 * section "Architecture: one command buffer per token").
 *
 *  fmt          one of qg_format.
 *  rows         N, the number of output rows; a stack of E equally shaped
 *               expert matrices is packed as rows = E * N_expert.
 *  K            inputs per row: a multiple of 64 (Q4), 32 (Q8, MXFP4,
 *               Q8_ROW) or of the group (AFFINE), 1 <= K <= 2^20.
 *  codes, scales, biases   canonical device buffers (layouts above); biases is
 *               required for Q4 and AFFINE and must be NULL otherwise.  Read
 *               only.
 *  packed       device buffer (16-B) receiving the packed layout, or NULL to
 *               query the size only (no device access at all then).
 *  packed_bytes in: capacity of `packed` (ignored when packed is NULL);
 *               out: bytes the layout needs.  Capacity below that -> QG_ESIZE.
 *  stream       hipStream_t.
 * Errors: QG_EINVAL (NULL codes/scales/packed_bytes, bias presence wrong),
 * QG_ESHAPE, QG_EALIGN, QG_ESIZE, QG_EHIP.
 */
int qgemv_pack(int fmt, int64_t rows, int64_t K, const void *codes,
               const void *scales, const void *biases, void *packed,
               size_t *packed_bytes, void *stream);

/*
 * qgemv_run -- decode GEMV, one activation row: y[n] = sum_k w[n][k] x[k]
 * (the product batch-one decode spends its time in; Uzu page, "Why batch-one
 * decoding is memory-bound").  Weights are dequantized in registers and
 * accumulated in fp32.
 *
 *  fmt          QG_FMT_Q4_ASYM_G64, QG_FMT_MXFP4_G32, QG_FMT_Q8_ROW or an
 *               affine-family code (Q8 -> QG_EUNSUPPORTED; use
 *               qgemm_skinny_run with M = 1).
 *  packed, packed_bytes   from qgemv_pack with the same (fmt, N, K); 16-B.
 *  N, K         output rows and inputs; K <= 24576 for this call.
 *  x            device bf16 [K], 16-B.  Read only.
 *  y            device [N] of the output type (bf16 or fp32), written.
 *  out_dtype    QG_OUT_BF16 or QG_OUT_F32.
 * Errors: QG_EINVAL, QG_ESHAPE, QG_EALIGN, QG_ESIZE, QG_EUNSUPPORTED, QG_EHIP.
 */
int qgemv_run(int fmt, const void *packed, size_t packed_bytes, int64_t N,
              int64_t K, const void *x, void *y, int out_dtype, void *stream);

/*
 * qgemm_skinny_run -- the skinny product Y[m][n] = sum_k w[n][k] X[m][k] for
 * M = 1..32 activation rows against the same weights, streamed once per call
 * (one verification pass over a 16- or 32-token draft; Uzu page, "Producing
 * several tokens from one model pass").  Runs on the MFMA matrix cores.
 *
 *  fmt          QG_FMT_Q4_ASYM_G64: X is bf16 [M][K], x_scales must be NULL.
 *               QG_FMT_Q8_SYM_G32: X is int8 [M][K] (from hadamard32_quant_run,
 *               so the weights must already be in the rotated basis) and
 *               x_scales fp32 [M] is the per-row activation scale.
 *               An affine-family code: X is bf16 [M][K], x_scales must be
 *               NULL (M = 1 runs the decode GEMV).
 *               Other formats -> QG_EUNSUPPORTED (MXFP4 and Q8_ROW are
 *               decode GEMVs: qgemv_run).
 *  packed, packed_bytes   from qgemv_pack with the same (fmt, N, K); 16-B.
 *  M            0..32.
 *  X            device [M][K], rows contiguous, 16-B.  Read only.
 *  Y            device output: [M][N] bf16 or fp32; for QG_OUT_I32_GROUPS
 *               (Q8 only) int32 [M][N][K/32], the exact group partials
 *               sum_{k in g} qw[n][k] * qx[m][k].
 * Errors: QG_EINVAL, QG_ESHAPE, QG_EALIGN, QG_ESIZE, QG_EUNSUPPORTED, QG_EHIP.
 */
int qgemm_skinny_run(int fmt, const void *packed, size_t packed_bytes,
                     int64_t M, int64_t N, int64_t K, const void *X,
                     const float *x_scales, void *Y, int out_dtype,
                     void *stream);

/*
 * hadamard32_quant_run -- on-the-fly int8 quantization of activations after a
 * block-diagonal randomized Hadamard transform (Uzu page, "How Uzu optimizes
 * bytes and tokens per pass"): for each row m and each block of 32
 * consecutive k, z = H32 (d . x) with H32 the +-1 Sylvester Hadamard matrix
 * (H[i][j] = (-1)^popcount(i & j)) and d the sign flips, applied before the
 * mixing.  Then per row: amax = max |z|, Xq = round-half-even(z * 127 / amax)
 * (computed in fp64; the sums are exact) and x_scales[m] = amax /
 * (127 * sqrt(32)) rounded to fp32, so that x_scales[m] * Xq approximates the
 * orthonormal rotation z / sqrt(32).  A zero row gives Xq = 0, scale 0.
 *
 *  X            device bf16 [M][K], 16-B.  Read only.
 *  signs        device int8 [K], 16-B, each +1 or -1 (other values are used
 *               as given).  Read only.
 *  M, K         M >= 0, K a positive multiple of 32.
 *  Xq           device int8 [M][K], 16-B, written.
 *  x_scales     device fp32 [M], written.
 * Errors: QG_EINVAL, QG_ESHAPE, QG_EALIGN, QG_EHIP.
 */
int hadamard32_quant_run(const void *X, const int8_t *signs, int64_t M,
                         int64_t K, int8_t *Xq, float *x_scales, void *stream);

/*
 * Bytes of workspace moe_expert_gemv_run needs for (top_k, H, F): the SwiGLU
 * activations h (fp32 [top_k][F]), the per-expert partial outputs (fp32
 * [top_k][H]) and a status word.  Pure host function.
 */
size_t qg_moe_workspace_bytes(int64_t top_k, int64_t H, int64_t F);

/*
 * moe_expert_gemv_run -- one token through the routed experts of one MoE
 * layer in MXFP4 (Deltafin / Kimi K3 page: the router selects the top-k
 * experts and only those are read; fused MXFP4 dequant + GEMV):
 *     for s < top_k with e = expert_ids[s]:
 *         g = Wgate[e] x,  u = Wup[e] x,  h = silu(g) * u,
 *     y = sum_s expert_w[s] * (Wdown[e] h).
 * g, u, h and the partial outputs are fp32; y is rounded once at the end.
 * expert_ids and expert_w stay on the device (no host round trip).  The
 * weighted sum is taken in slot order, so results are deterministic.
 *
 *  packed_gate, packed_up   qgemv_pack(MXFP4, rows = E * F, K = H), 16-B.
 *  packed_down              qgemv_pack(MXFP4, rows = E * H, K = F), 16-B.
 *  bytes_*      sizes from those qgemv_pack calls.
 *  E, H, F      experts, hidden size, expert FFN size; H and F positive
 *               multiples of 32; H <= 24576, F <= 12288.
 *  x            device bf16 [H], 16-B.  Read only.
 *  top_k        0..min(E, 64).
 *  expert_ids   device int32 [top_k]; an id outside [0, E) contributes 0.
 *               The call rewrites a status word (uint32 at byte offset
 *               4 * top_k * (F + H) of the workspace): 1 if any id was out
 *               of range, else 0.
 *  expert_w     device fp32 [top_k] router weights.
 *  workspace    device buffer (16-B) of at least qg_moe_workspace_bytes bytes;
 *               its contents are scratch, overwritten by every call.
 *  y            device [H] bf16 or fp32, written.
 * Errors: QG_EINVAL, QG_ESHAPE, QG_EALIGN, QG_ESIZE, QG_EUNSUPPORTED, QG_EHIP.
 */
int moe_expert_gemv_run(const void *packed_gate, const void *packed_up,
                        const void *packed_down, size_t bytes_gate,
                        size_t bytes_up, size_t bytes_down, int64_t E,
                        int64_t H, int64_t F, const void *x, int top_k,
                        const int32_t *expert_ids, const float *expert_w,
                        void *workspace, size_t workspace_bytes, void *y,
                        int out_dtype, void *stream);

/*
 * Bytes of workspace moe_expert_skinny_run needs for (T, top_k, H, F), with
 * P = T * top_k (position, slot) pairs: h (fp32 [P][F]), the per-pair partial
 * outputs (fp32 [P][H]), a 16-byte header (status word first) and the
 * expert groups (32 bytes per pair).  Pure host function.
 */
size_t qg_moe_skinny_workspace_bytes(int64_t T, int64_t top_k, int64_t H,
                                     int64_t F);

/* The largest workspace moe_expert_gemv_run_noalloc serves (its
 * qg_moe_workspace_bytes(top_k, H, F) must not exceed this): 2 MiB, e.g.
 * top_k = 16 with H + F up to 32767.  The library holds one array of this
 * size on each GPU it runs the call on, until the process ends. */
#define QG_MOE_NOALLOC_SCRATCH_BYTES ((size_t)2 << 20)

/*
 * moe_expert_gemv_run_noalloc -- moe_expert_gemv_run for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The same computation, kernels and
 * results as moe_expert_gemv_run (bit for bit); instead of a caller
 * workspace it uses the library's array of QG_MOE_NOALLOC_SCRATCH_BYTES on
 * the current device.  It allocates and frees nothing (the array's device
 * address is looked up once per device, on the first call there).
 *
 *  status       optional device uint32 (4-B aligned), written: 1 if any id
 *               was out of range, else 0.  NULL: not reported.
 *  other arguments as in moe_expert_gemv_run (no workspace).
 * The array keeps the previous call's contents; every call writes whatever
 * it reads from it first, so nothing needs clearing.  All calls on one GPU
 * share the one array: calls that overlap on a GPU (concurrent streams or
 * host threads) race on it and must be serialized by the caller.
 * Errors: those of moe_expert_gemv_run; QG_ESIZE when
 * qg_moe_workspace_bytes(top_k, H, F) > QG_MOE_NOALLOC_SCRATCH_BYTES;
 * QG_EUNSUPPORTED on a device index of 64 or more.
 */
int moe_expert_gemv_run_noalloc(const void *packed_gate, const void *packed_up,
                                const void *packed_down, size_t bytes_gate,
                                size_t bytes_up, size_t bytes_down, int64_t E,
                                int64_t H, int64_t F, const void *x, int top_k,
                                const int32_t *expert_ids, const float *expert_w,
                                uint32_t *status, void *y, int out_dtype, void *stream);

/*
 * moe_expert_skinny_run -- T positions (a verification tile of draft tokens)
 * through the routed experts of one MoE layer in MXFP4, each position with
 * its own router output (Deltafin / Kimi K3 page, "How it works": only the
 * selected experts are read):
 *     for t < T, s < top_k with e = expert_ids[t][s]:
 *         g = Wgate[e] X[t],  u = Wup[e] X[t],  h = silu(g) * u,
 *     Y[t] = sum_s expert_w[t][s] * (Wdown[e] h).
 * Each row of Y is what moe_expert_gemv_run returns for X[t], ids[t], w[t],
 * up to rounding.  The weights of an expert chosen by several positions are
 * read once for up to four of them, so a pass reads about the union of the
 * positions' experts.  g, u, h and the partial outputs are fp32 (h enters
 * the down projection as a bf16 pair hi + lo, relative error <= 2^-16); Y is
 * rounded once at the end; every sum is taken in a fixed order, so results
 * are deterministic.  The ids stay on the device.
 *
 *  packed_gate, packed_up, packed_down, bytes_*, E, H, F
 *               as for moe_expert_gemv_run.
 *  T            positions, 1..32, with T * top_k <= 2048.
 *  X            device bf16 [T][H], 16-B.  Read only.
 *  top_k        0..min(E, 64).
 *  expert_ids   device int32 [T][top_k]; an id outside [0, E) contributes 0.
 *               The call rewrites a status word (uint32 at byte offset
 *               4 * T * top_k * (F + H) of the workspace): 1 if any id was
 *               out of range, else 0.
 *  expert_w     device fp32 [T][top_k] router weights.
 *  workspace    device buffer (16-B) of at least qg_moe_skinny_workspace_bytes
 *               bytes; scratch, overwritten by every call.
 *  Y            device [T][H] bf16 or fp32, written.
 * Errors: QG_EINVAL, QG_ESHAPE, QG_EALIGN, QG_ESIZE, QG_EUNSUPPORTED, QG_EHIP.
 */
int moe_expert_skinny_run(const void *packed_gate, const void *packed_up,
                          const void *packed_down, size_t bytes_gate,
                          size_t bytes_up, size_t bytes_down, int64_t E,
                          int64_t H, int64_t F, int64_t T, const void *X,
                          int top_k, const int32_t *expert_ids,
                          const float *expert_w, void *workspace,
                          size_t workspace_bytes, void *Y, int out_dtype,
                          void *stream);

/*
 * Grouped launches: many independent products in one kernel launch.
 *
 * A decode step runs every projection of the model once per token; issuing
 * them as one piece of GPU work, rather than one launch each, is what the
 * "one command buffer per token" design of "MLX Runner: An Inference Engine
 * You Can Read" (section "Architecture: one command buffer per token") does
 * on Apple GPUs.  Here the products are described once, on the host, by an
 * array of qg_gemv_desc; qg_batch_plan_build validates them, balances the
 * work across the GPU by bytes and writes a work list into caller-owned
 * device memory; qg_batch_run then enqueues a single persistent kernel that
 * computes every product of the list.  The products must be independent (no
 * output of one is an input of another within the list).
 */
typedef struct qg_gemv_desc {
    const void *packed;   /* from qgemv_pack(fmt, N, K); 16-B */
    size_t packed_bytes;
    int64_t N, K;
    const void *x;        /* device bf16 [M][K], 16-B; read only */
    void *y;              /* device [M][N] of the plan's output type; written */
} qg_gemv_desc;

/* Kernel family of a grouped launch.  Q4 products have two: the VALU GEMV
 * kernel (codes unpacked in registers, one v_dot2 chain per activation row;
 * 1..4 rows) and the bf16 MFMA kernel (16x16x32 tiles of 16 or 32 rows,
 * whatever M is).  QG_KERNEL_AUTO takes the one measured faster on MI355X:
 * VALU for M = 1, MFMA for M >= 2 (at M = 2 the MFMA pass over a decode
 * step's weights already takes 0.671 ms against 0.761 ms on the VALU).  The
 * others force a family, e.g. to measure both; results differ between the
 * families only by fp32 rounding order.  Affine products have one kernel per
 * M: at M = 1 the GEMV kernel of qgemv_run (QG_KERNEL_AUTO or
 * QG_KERNEL_VALU), for more rows the MFMA kernel of qgemm_skinny_run
 * (QG_KERNEL_AUTO or QG_KERNEL_MFMA); int8 row-scale GEMVs (M = 1) only the
 * kernel of qgemv_run (QG_KERNEL_AUTO or QG_KERNEL_VALU). */
typedef enum {
    QG_KERNEL_AUTO = 0,
    QG_KERNEL_VALU = 1,   /* M <= 4, else QG_EUNSUPPORTED */
    QG_KERNEL_MFMA = 2
} qg_kernel;

/* Launch plan: plain host data, filled by qg_batch_plan_build and consumed
 * by qg_batch_run.  The fields are not meant to be edited; `kernel` holds
 * the family chosen (never QG_KERNEL_AUTO). */
typedef struct qg_batch_plan {
    int32_t fmt, M, count, out_dtype;
    int32_t grid, kmax, kernel, reserved1;
    const void *worklist;
    size_t worklist_bytes;
} qg_batch_plan;

/* Device bytes of the work list for `count` products (host function). */
size_t qg_batch_worklist_bytes(int32_t count);

/*
 * qg_batch_plan_build -- validate `count` product descriptors and write their
 * work list to `worklist`.
 *
 *  fmt          QG_FMT_Q4_ASYM_G64; a QG_FMT_AFFINE(bits, group, bf16) code
 *               (M = 1: the affine decode GEMV, QG_KERNEL_MFMA ->
 *               QG_EUNSUPPORTED; M > 1: the affine skinny product on the
 *               bf16 MFMA, QG_KERNEL_VALU -> QG_EUNSUPPORTED); or
 *               QG_FMT_Q8_ROW (M = 1 only, the weight-only int8 GEMV; M > 1 or
 *               QG_KERNEL_MFMA -> QG_EUNSUPPORTED).  Other formats ->
 *               QG_EUNSUPPORTED.  Every descriptor's packed buffer is of `fmt`.
 *  M            activation rows of every product: 1 (decode GEMVs, K <= 24576
 *               each) or 2..32 (a verification pass; Q4 and affine).
 *  count        1..65536 descriptors in `descs` (host array, read only; it
 *               need not outlive the call).
 *  out_dtype    QG_OUT_BF16 or QG_OUT_F32, for every product.
 *  kernel       a qg_kernel: QG_KERNEL_AUTO, or a family to force.
 *  worklist     device buffer (16-B) of at least qg_batch_worklist_bytes(count)
 *               bytes; written asynchronously on `stream`, then read by every
 *               qg_batch_run of this plan, so it must stay allocated and
 *               unmodified while the plan is in use.
 *  plan         host struct receiving the plan.
 * Errors: QG_EINVAL (also an unknown kernel), QG_ESHAPE, QG_EALIGN, QG_ESIZE
 * (a descriptor's packed_bytes, or worklist_bytes), QG_EUNSUPPORTED (also
 * QG_KERNEL_VALU with M > 4), QG_EHIP.
 */
int qg_batch_plan_build(int fmt, int64_t M, int32_t count, const qg_gemv_desc *descs,
                        int out_dtype, int kernel, void *worklist, size_t worklist_bytes,
                        qg_batch_plan *plan, void *stream);

/*
 * qg_batch_run -- enqueue one kernel computing every product of the plan:
 * Y_i = X_i W_i^T (y_i = W_i x_i for M = 1).  Every output equals the single
 * call's bit for bit: qgemv_run's at M = 1 (every format), and for M > 1
 * qgemm_skinny_run's for affine products, and for Q4 products where that
 * call takes the streaming kernel too (matrices of at least 2 * 16 rowblocks
 * per CU, such as an output head); smaller single Q4 products split K over
 * waves and differ from the grouped ones by fp32 rounding order only.  The
 * buffers named in the descriptors must still be valid.  Safe to capture in
 * a HIP graph.
 * Errors: QG_EINVAL (NULL or malformed plan), QG_EHIP.
 */
int qg_batch_run(const qg_batch_plan *plan, void *stream);

/*
 * qg_plain_read -- measurement utility: read `bytes` of the device buffer
 * `buf` once with plain streaming loads (workgroup j of `grid` takes the
 * j-th contiguous share, non-temporal 16-byte loads) and write the XOR of
 * the words each workgroup read to sink[j].  Its rate is the practical read
 * ceiling of this GPU, against which the kernels above are also rated (both
 * "MLX Runner: An Inference Engine You Can Read", section "Optimized against
 * a known ceiling", and the Uzu page, section "Why batch-one decoding is
 * memory-bound", rate decode by bandwidth over bytes).
 *
 *  buf      device, 16-B aligned; read only.  bytes: a multiple of 16 (0: no-op).
 *  sink     device uint32 [grid], 4-B aligned; written.
 *  grid     workgroups, 1..65536.
 * Errors: QG_EINVAL (NULL pointer), QG_ESHAPE (bytes % 16, grid), QG_EALIGN,
 * QG_EHIP.
 */
int qg_plain_read(const void *buf, size_t bytes, uint32_t *sink, int grid, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
