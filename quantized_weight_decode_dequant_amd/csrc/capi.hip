// C ABI of the library (declared in include/qgemv.h).  Every entry point
// validates its arguments on the host before any HIP call -- model inputs are
// checked explicitly before anything reaches the GPU and unsupported feature
// combinations return an error instead of being ignored ("MLX Runner: An
// Inference Engine You Can Read", section "Untrusted input, verified
// output") -- then enqueues its kernels on the caller's stream and returns.
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/qgemv.h"
#include "qg_internal.h"

namespace {

using namespace qg;

constexpr int64_t K_MAX = int64_t(1) << 20;
constexpr int64_t N_MAX = int64_t(1) << 30;
constexpr int64_t GEMV_K_MAX = 24576;  // x staged whole in LDS
constexpr int64_t MOE_H_MAX = 24576;
constexpr int64_t MOE_F_MAX = 12288;   // h staged whole in LDS as fp32
constexpr int MOE_TOPK_MAX = 64;
constexpr int M_MAX = 32;
// Q4 products with at most this many activation rows run on the VALU GEMV
// kernel by default; more rows go to the bf16 MFMA kernels.  Measured on
// MI355X over a decode step's weights: M = 1 takes 0.643 ms on the VALU and
// 0.654 ms on MFMA, M = 2 0.761 and 0.671 ms, M = 4 1.181 and 0.701 ms, so
// MFMA from M = 2 on.
constexpr int Q4_VALU_ROWS_MAX = 1;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int format_group(int fmt) {
    switch (fmt) {
    case QG_FMT_Q4_ASYM_G64: return 64;
    case QG_FMT_Q8_SYM_G32: return 32;
    case QG_FMT_MXFP4_G32: return 32;
    case QG_FMT_Q8_ROW: return 32;
    default: return affine_decode(fmt).group;
    }
}

size_t packed_bytes_for(int fmt, int64_t N, int64_t K) {
    switch (fmt) {
    case QG_FMT_Q4_ASYM_G64: return q4_packed_bytes(N, K);
    case QG_FMT_Q8_SYM_G32: return q8_packed_bytes(N, K);
    case QG_FMT_MXFP4_G32: return fp4_packed_bytes(N, K);
    case QG_FMT_Q8_ROW: return q8row_packed_bytes(N, K);
    default: {
        const AffineFmt a = affine_decode(fmt);
        return a.bits ? affine_packed_bytes(a.bits, a.group, N, K) : 0;
    }
    }
}

// shape rules shared by every weight matrix
int check_matrix(int fmt, int64_t N, int64_t K) {
    const int g = format_group(fmt);
    if (g == 0) return QG_EINVAL;
    if (N < 0 || N > N_MAX || K <= 0 || K > K_MAX || K % g != 0) return QG_ESHAPE;
    return QG_OK;
}

std::atomic<int> g_cus[64];

int device_cus(int *cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QG_EHIP;
    if (dev < 0 || dev >= 64) dev = 0;
    int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c <= 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return QG_EHIP;
        if (c <= 0) c = 1;
        g_cus[dev].store(c, std::memory_order_relaxed);
    }
    *cus = c;
    return QG_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? QG_OK : QG_EHIP; }

}  // namespace

extern "C" {

const char *qg_status_string(int status) {
    switch (status) {
    case QG_OK: return "QG_OK";
    case QG_EINVAL: return "QG_EINVAL: null pointer or unknown enum value";
    case QG_ESHAPE: return "QG_ESHAPE: dimension out of range";
    case QG_EALIGN: return "QG_EALIGN: device pointer misaligned";
    case QG_ESIZE: return "QG_ESIZE: buffer size does not match the layout";
    case QG_EUNSUPPORTED: return "QG_EUNSUPPORTED: format/output/entry point combination not provided";
    case QG_EHIP: return "QG_EHIP: HIP runtime error";
    case QG_EINTERNAL: return "QG_EINTERNAL: internal error";
    default: return "unknown qg_status";
    }
}

int qg_version(void) { return 100; }

int qgemv_pack(int fmt, int64_t rows, int64_t K, const void *codes, const void *scales,
               const void *biases, void *packed, size_t *packed_bytes, void *stream) {
    try {
        if (!packed_bytes) return QG_EINVAL;
        int st = check_matrix(fmt, rows, K);
        if (st != QG_OK) return st;
        const size_t need = packed_bytes_for(fmt, rows, K);
        if (!packed) {
            *packed_bytes = need;
            return QG_OK;
        }
        if (!codes || !scales) return QG_EINVAL;
        const AffineFmt aff = affine_decode(fmt);
        if ((fmt == QG_FMT_Q4_ASYM_G64 || aff.bits) != (biases != nullptr)) return QG_EINVAL;
        if (*packed_bytes < need) {
            *packed_bytes = need;
            return QG_ESIZE;
        }
        *packed_bytes = need;
        if (!aligned(packed, 16) || !aligned(codes, 16) ||
            !aligned(scales, fmt == QG_FMT_Q8_ROW ? 4 : 2) || (biases && !aligned(biases, 2)))
            return QG_EALIGN;
        if (rows == 0) return QG_OK;
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        uint8_t *out = reinterpret_cast<uint8_t *>(packed);
        switch (fmt) {
        case QG_FMT_Q4_ASYM_G64:
            return hip_status(launch_pack_q4(reinterpret_cast<const uint32_t *>(codes),
                                             reinterpret_cast<const uint16_t *>(scales),
                                             reinterpret_cast<const uint16_t *>(biases), rows, K,
                                             out, s));
        case QG_FMT_Q8_SYM_G32:
            return hip_status(launch_pack_q8(reinterpret_cast<const int8_t *>(codes),
                                             reinterpret_cast<const uint16_t *>(scales), rows, K,
                                             out, s));
        case QG_FMT_MXFP4_G32:
            return hip_status(launch_pack_fp4(reinterpret_cast<const uint8_t *>(codes),
                                              reinterpret_cast<const uint8_t *>(scales), rows, K,
                                              out, s));
        case QG_FMT_Q8_ROW:
            return hip_status(launch_pack_q8row(reinterpret_cast<const int8_t *>(codes),
                                                reinterpret_cast<const float *>(scales), rows, K,
                                                out, s));
        default:
            return hip_status(launch_pack_affine(reinterpret_cast<const uint8_t *>(codes),
                                                 reinterpret_cast<const uint16_t *>(scales),
                                                 reinterpret_cast<const uint16_t *>(biases),
                                                 aff.bits, aff.group, rows, K, out, s));
        }
    } catch (...) {
        return QG_EINTERNAL;
    }
}

int qgemv_run(int fmt, const void *packed, size_t packed_bytes, int64_t N, int64_t K,
              const void *x, void *y, int out_dtype, void *stream) {
    try {
        if (out_dtype != QG_OUT_BF16 && out_dtype != QG_OUT_F32 && out_dtype != QG_OUT_I32_GROUPS)
            return QG_EINVAL;
        int st = check_matrix(fmt, N, K);
        if (st != QG_OK) return st;
        if (fmt == QG_FMT_Q8_SYM_G32 || out_dtype == QG_OUT_I32_GROUPS) return QG_EUNSUPPORTED;
        if (!packed || !x || !y) return QG_EINVAL;
        if (K > GEMV_K_MAX) return QG_ESHAPE;
        if (packed_bytes != packed_bytes_for(fmt, N, K)) return QG_ESIZE;
        if (!aligned(packed, 16) || !aligned(x, 16) ||
            !aligned(y, out_dtype == QG_OUT_F32 ? 4 : 2))
            return QG_EALIGN;
        if (N == 0) return QG_OK;
        int cus = 0;
        if ((st = device_cus(&cus)) != QG_OK) return st;
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        const bool f32 = out_dtype == QG_OUT_F32;
        const uint8_t *p = reinterpret_cast<const uint8_t *>(packed);
        const uint16_t *xx = reinterpret_cast<const uint16_t *>(x);
        if (fmt == QG_FMT_Q4_ASYM_G64) return hip_status(launch_q4_gemv(p, xx, y, 1, N, K, f32, cus, s));
        if (fmt == QG_FMT_Q8_ROW) return hip_status(launch_q8row_gemv(p, xx, y, N, K, f32, cus, s));
        if (fmt == QG_FMT_MXFP4_G32) return hip_status(launch_fp4_gemv(p, xx, y, N, K, f32, cus, s));
        const AffineFmt a = affine_decode(fmt);
        return hip_status(launch_affine_gemv(p, xx, y, a.bits, a.group, a.bf16 != 0, N, K, f32,
                                             cus, s));
    } catch (...) {
        return QG_EINTERNAL;
    }
}

int qgemm_skinny_run(int fmt, const void *packed, size_t packed_bytes, int64_t M, int64_t N,
                     int64_t K, const void *X, const float *x_scales, void *Y, int out_dtype,
                     void *stream) {
    try {
        if (out_dtype != QG_OUT_BF16 && out_dtype != QG_OUT_F32 && out_dtype != QG_OUT_I32_GROUPS)
            return QG_EINVAL;
        int st = check_matrix(fmt, N, K);
        if (st != QG_OK) return st;
        const AffineFmt aff = affine_decode(fmt);
        if (fmt != QG_FMT_Q4_ASYM_G64 && fmt != QG_FMT_Q8_SYM_G32 && !aff.bits)
            return QG_EUNSUPPORTED;
        if (fmt != QG_FMT_Q8_SYM_G32 && out_dtype == QG_OUT_I32_GROUPS) return QG_EUNSUPPORTED;
        if (M < 0 || M > M_MAX) return QG_ESHAPE;
        if (!packed || !X || !Y) return QG_EINVAL;
        if (fmt == QG_FMT_Q8_SYM_G32 && out_dtype != QG_OUT_I32_GROUPS && !x_scales) return QG_EINVAL;
        if (fmt != QG_FMT_Q8_SYM_G32 && x_scales) return QG_EINVAL;
        if (packed_bytes != packed_bytes_for(fmt, N, K)) return QG_ESIZE;
        const size_t yal = out_dtype == QG_OUT_BF16 ? 2 : 4;
        if (!aligned(packed, 16) || !aligned(X, 16) || !aligned(Y, yal) ||
            (x_scales && !aligned(x_scales, 4)))
            return QG_EALIGN;
        if (M == 0 || N == 0) return QG_OK;
        int cus = 0;
        if ((st = device_cus(&cus)) != QG_OK) return st;
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        const uint8_t *p = reinterpret_cast<const uint8_t *>(packed);
        if (fmt == QG_FMT_Q4_ASYM_G64) {
            const uint16_t *xx = reinterpret_cast<const uint16_t *>(X);
            const bool f32 = out_dtype == QG_OUT_F32;
            if (M <= Q4_VALU_ROWS_MAX)
                return hip_status(launch_q4_gemv(p, xx, Y, M, N, K, f32, cus, s));
            if (q4_skinny_stream_fits(N, cus))
                return hip_status(launch_q4_skinny_stream(p, xx, Y, M, N, K, f32, cus, s));
            return hip_status(launch_q4_skinny(p, xx, Y, M, N, K, f32, cus, s));
        }
        if (aff.bits) {
            const uint16_t *xx = reinterpret_cast<const uint16_t *>(X);
            const bool f32 = out_dtype == QG_OUT_F32;
            if (M == 1)
                return hip_status(launch_affine_gemv(p, xx, Y, aff.bits, aff.group, aff.bf16 != 0,
                                                     N, K, f32, cus, s));
            return hip_status(launch_affine_skinny(p, xx, Y, aff.bits, aff.group, aff.bf16 != 0,
                                                   M, N, K, f32, cus, s));
        }
        const int mode = out_dtype == QG_OUT_BF16 ? 0 : (out_dtype == QG_OUT_F32 ? 1 : 2);
        return hip_status(launch_q8_skinny(p, reinterpret_cast<const int8_t *>(X), x_scales, Y, M,
                                           N, K, mode, cus, s));
    } catch (...) {
        return QG_EINTERNAL;
    }
}

int hadamard32_quant_run(const void *X, const int8_t *signs, int64_t M, int64_t K, int8_t *Xq,
                         float *x_scales, void *stream) {
    try {
        if (!X || !signs || !Xq || !x_scales) return QG_EINVAL;
        if (M < 0 || M > N_MAX || K <= 0 || K > K_MAX || K % 32 != 0) return QG_ESHAPE;
        if (!aligned(X, 16) || !aligned(signs, 16) || !aligned(Xq, 16) || !aligned(x_scales, 4))
            return QG_EALIGN;
        if (M == 0) return QG_OK;
        // 127 * sqrt(32): the Hadamard's global 1/sqrt(32) folded into the scale
        const double denom = 127.0 * std::sqrt(32.0);
        return hip_status(launch_had32_quant(reinterpret_cast<const uint16_t *>(X), signs, M, K,
                                             Xq, x_scales, denom,
                                             reinterpret_cast<hipStream_t>(stream)));
    } catch (...) {
        return QG_EINTERNAL;
    }
}

size_t qg_moe_workspace_bytes(int64_t top_k, int64_t H, int64_t F) {
    if (top_k < 0 || H < 0 || F < 0) return 0;
    return (size_t)4 * (size_t)top_k * (size_t)(F + H) + 16;
}

size_t qg_moe_skinny_workspace_bytes(int64_t T, int64_t top_k, int64_t H, int64_t F) {
    if (T < 0 || top_k < 0 || H < 0 || F < 0) return 0;
    const size_t P = (size_t)T * (size_t)top_k;
    return (size_t)4 * P * (size_t)(F + H) + 16 + (size_t)32 * P;
}

}  // extern "C"

namespace {

// Checks shared by the MoE entry points (everything but the activations,
// the workspace size and the output).
int moe_validate(const void *packed_gate, const void *packed_up, const void *packed_down,
                 size_t bytes_gate, size_t bytes_up, size_t bytes_down, int64_t E, int64_t H,
                 int64_t F, int top_k, const int32_t *expert_ids, const float *expert_w,
                 int out_dtype) {
    if (out_dtype != QG_OUT_BF16 && out_dtype != QG_OUT_F32 && out_dtype != QG_OUT_I32_GROUPS)
        return QG_EINVAL;
    if (out_dtype == QG_OUT_I32_GROUPS) return QG_EUNSUPPORTED;
    if (E < 1 || H < 32 || F < 32 || H % 32 || F % 32 || H > MOE_H_MAX || F > MOE_F_MAX ||
        E * F > N_MAX || E * H > N_MAX)
        return QG_ESHAPE;
    if (top_k < 0 || top_k > MOE_TOPK_MAX || top_k > E) return QG_ESHAPE;
    if (!packed_gate || !packed_up || !packed_down) return QG_EINVAL;
    if (top_k > 0 && (!expert_ids || !expert_w)) return QG_EINVAL;
    if (bytes_gate != fp4_packed_bytes(E * F, H) || bytes_up != fp4_packed_bytes(E * F, H) ||
        bytes_down != fp4_packed_bytes(E * H, F))
        return QG_ESIZE;
    return QG_OK;
}

}  // namespace

extern "C" {

int moe_expert_gemv_run(const void *packed_gate, const void *packed_up, const void *packed_down,
                        size_t bytes_gate, size_t bytes_up, size_t bytes_down, int64_t E,
                        int64_t H, int64_t F, const void *x, int top_k,
                        const int32_t *expert_ids, const float *expert_w, void *workspace,
                        size_t workspace_bytes, void *y, int out_dtype, void *stream) {
    try {
        int st = moe_validate(packed_gate, packed_up, packed_down, bytes_gate, bytes_up,
                              bytes_down, E, H, F, top_k, expert_ids, expert_w, out_dtype);
        if (st != QG_OK) return st;
        if (!workspace) return QG_EINVAL;
        if (!x || !y) return QG_EINVAL;
        if (workspace_bytes < qg_moe_workspace_bytes(top_k, H, F)) return QG_ESIZE;
        if (!aligned(packed_gate, 16) || !aligned(packed_up, 16) || !aligned(packed_down, 16) ||
            !aligned(x, 16) || !aligned(workspace, 16) ||
            !aligned(y, out_dtype == QG_OUT_F32 ? 4 : 2) ||
            (expert_ids && !aligned(expert_ids, 4)) || (expert_w && !aligned(expert_w, 4)))
            return QG_EALIGN;
        int cus = 0;
        st = device_cus(&cus);
        if (st != QG_OK) return st;
        return hip_status(launch_moe(reinterpret_cast<const uint8_t *>(packed_gate),
                                     reinterpret_cast<const uint8_t *>(packed_up),
                                     reinterpret_cast<const uint8_t *>(packed_down), E, H, F,
                                     reinterpret_cast<const uint16_t *>(x), top_k, expert_ids,
                                     expert_w, reinterpret_cast<uint8_t *>(workspace), y,
                                     out_dtype == QG_OUT_F32, cus,
                                     reinterpret_cast<hipStream_t>(stream)));
    } catch (...) {
        return QG_EINTERNAL;
    }
}

}  // extern "C"

// ---- the allocation-free MoE call
// Its workspace is this array, one per GPU the library runs on (each device
// holds its own copy, at its own address, until the process ends).  In host
// code `qg_moe_scratch` names a host-side stand-in, not device memory: its
// device address comes from hipGetSymbolAddress, looked up once per device
// with that device current, and only that address is passed to kernels.
static __device__ __align__(256) unsigned char qg_moe_scratch[QG_MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int SCRATCH_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[SCRATCH_DEVICES];  // device address per device, null until looked up

int moe_scratch_ptr(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QG_EHIP;
    if (dev < 0 || dev >= SCRATCH_DEVICES) return QG_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(qg_moe_scratch)) != hipSuccess || !p)
            return QG_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QG_OK;
}

}  // namespace

extern "C" {

int moe_expert_gemv_run_noalloc(const void *packed_gate, const void *packed_up,
                                const void *packed_down, size_t bytes_gate, size_t bytes_up,
                                size_t bytes_down, int64_t E, int64_t H, int64_t F,
                                const void *x, int top_k, const int32_t *expert_ids,
                                const float *expert_w, uint32_t *status, void *y, int out_dtype,
                                void *stream) {
    try {
        int st = moe_validate(packed_gate, packed_up, packed_down, bytes_gate, bytes_up,
                              bytes_down, E, H, F, top_k, expert_ids, expert_w, out_dtype);
        if (st != QG_OK) return st;
        if (!x || !y) return QG_EINVAL;
        if (qg_moe_workspace_bytes(top_k, H, F) > QG_MOE_NOALLOC_SCRATCH_BYTES) return QG_ESIZE;
        if (!aligned(packed_gate, 16) || !aligned(packed_up, 16) || !aligned(packed_down, 16) ||
            !aligned(x, 16) || !aligned(y, out_dtype == QG_OUT_F32 ? 4 : 2) ||
            (status && !aligned(status, 4)) || (expert_ids && !aligned(expert_ids, 4)) ||
            (expert_w && !aligned(expert_w, 4)))
            return QG_EALIGN;
        int cus = 0;
        if ((st = device_cus(&cus)) != QG_OK) return st;
        void *ws = nullptr;
        if ((st = moe_scratch_ptr(&ws)) != QG_OK) return st;
        return hip_status(launch_moe(reinterpret_cast<const uint8_t *>(packed_gate),
                                     reinterpret_cast<const uint8_t *>(packed_up),
                                     reinterpret_cast<const uint8_t *>(packed_down), E, H, F,
                                     reinterpret_cast<const uint16_t *>(x), top_k, expert_ids,
                                     expert_w, reinterpret_cast<uint8_t *>(ws), y,
                                     out_dtype == QG_OUT_F32, cus,
                                     reinterpret_cast<hipStream_t>(stream),
                                     reinterpret_cast<unsigned *>(status)));
    } catch (...) {
        return QG_EINTERNAL;
    }
}

int moe_expert_skinny_run(const void *packed_gate, const void *packed_up,
                          const void *packed_down, size_t bytes_gate, size_t bytes_up,
                          size_t bytes_down, int64_t E, int64_t H, int64_t F, int64_t T,
                          const void *X, int top_k, const int32_t *expert_ids,
                          const float *expert_w, void *workspace, size_t workspace_bytes,
                          void *Y, int out_dtype, void *stream) {
    try {
        int st = moe_validate(packed_gate, packed_up, packed_down, bytes_gate, bytes_up,
                              bytes_down, E, H, F, top_k, expert_ids, expert_w, out_dtype);
        if (st != QG_OK) return st;
        if (!workspace) return QG_EINVAL;
        if (T < 1 || T > M_MAX || T * top_k > MOE_PAIRS_MAX) return QG_ESHAPE;
        if (!X || !Y) return QG_EINVAL;
        if (workspace_bytes < qg_moe_skinny_workspace_bytes(T, top_k, H, F)) return QG_ESIZE;
        if (!aligned(packed_gate, 16) || !aligned(packed_up, 16) || !aligned(packed_down, 16) ||
            !aligned(X, 16) || !aligned(workspace, 16) ||
            !aligned(Y, out_dtype == QG_OUT_F32 ? 4 : 2) ||
            (expert_ids && !aligned(expert_ids, 4)) || (expert_w && !aligned(expert_w, 4)))
            return QG_EALIGN;
        int cus = 0;
        st = device_cus(&cus);
        if (st != QG_OK) return st;
        return hip_status(launch_moe_skinny(
            reinterpret_cast<const uint8_t *>(packed_gate),
            reinterpret_cast<const uint8_t *>(packed_up),
            reinterpret_cast<const uint8_t *>(packed_down), E, H, F, (int)T,
            reinterpret_cast<const uint16_t *>(X), top_k, expert_ids, expert_w,
            reinterpret_cast<uint8_t *>(workspace), Y, out_dtype == QG_OUT_F32, cus,
            reinterpret_cast<hipStream_t>(stream)));
    } catch (...) {
        return QG_EINTERNAL;
    }
}

size_t qg_batch_worklist_bytes(int32_t count) {
    if (count < 0) return 0;
    return (size_t)WL_HEADER_BYTES + sizeof(WorkItem) * (size_t)count +
           sizeof(WorkStart) * (size_t)(WL_GRID_MAX + 1);
}

int qg_batch_plan_build(int fmt, int64_t M, int32_t count, const qg_gemv_desc *descs,
                        int out_dtype, int kernel, void *worklist, size_t worklist_bytes,
                        qg_batch_plan *plan, void *stream) {
    try {
        if (!descs || !worklist || !plan) return QG_EINVAL;
        if (kernel != QG_KERNEL_AUTO && kernel != QG_KERNEL_VALU && kernel != QG_KERNEL_MFMA)
            return QG_EINVAL;
        if (out_dtype != QG_OUT_BF16 && out_dtype != QG_OUT_F32) {
            if (out_dtype == QG_OUT_I32_GROUPS) return QG_EUNSUPPORTED;
            return QG_EINVAL;
        }
        if (format_group(fmt) == 0) return QG_EINVAL;
        const AffineFmt aff = affine_decode(fmt);
        const bool q8row = fmt == QG_FMT_Q8_ROW;
        if (fmt != QG_FMT_Q4_ASYM_G64 && !aff.bits && !q8row) return QG_EUNSUPPORTED;
        if (M < 1 || M > M_MAX || count < 1 || count > 65536) return QG_ESHAPE;
        if (q8row) {
            // the weight-only int8 GEMV: one activation row
            if (M != 1 || kernel == QG_KERNEL_MFMA) return QG_EUNSUPPORTED;
            kernel = QG_KERNEL_VALU;
        }
        if (aff.bits) {
            // affine products: the decode GEMV at M = 1, the MFMA skinny
            // product for more rows
            if (M == 1) {
                if (kernel == QG_KERNEL_MFMA) return QG_EUNSUPPORTED;
                kernel = QG_KERNEL_VALU;
            } else {
                if (kernel == QG_KERNEL_VALU) return QG_EUNSUPPORTED;
                kernel = QG_KERNEL_MFMA;
            }
        }
        if (kernel == QG_KERNEL_AUTO) kernel = M <= Q4_VALU_ROWS_MAX ? QG_KERNEL_VALU : QG_KERNEL_MFMA;
        if (kernel == QG_KERNEL_VALU && M > q4_gemv_rows_max()) return QG_EUNSUPPORTED;
        if (worklist_bytes < qg_batch_worklist_bytes(count)) return QG_ESIZE;
        if (!aligned(worklist, 16)) return QG_EALIGN;
        const size_t yal = out_dtype == QG_OUT_F32 ? 4 : 2;
        int64_t kmax = 0;
        for (int32_t i = 0; i < count; ++i) {
            const qg_gemv_desc &d = descs[i];
            int st = check_matrix(fmt, d.N, d.K);
            if (st != QG_OK) return st;
            if (d.N < 1) return QG_ESHAPE;
            if (M == 1 && d.K > GEMV_K_MAX) return QG_ESHAPE;
            if (!d.packed || !d.x || !d.y) return QG_EINVAL;
            if (d.packed_bytes != packed_bytes_for(fmt, d.N, d.K)) return QG_ESIZE;
            if (!aligned(d.packed, 16) || !aligned(d.x, 16) || !aligned(d.y, yal)) return QG_EALIGN;
            if (d.K > kmax) kmax = d.K;
        }
        int cus = 0;
        int st = device_cus(&cus);
        if (st != QG_OK) return st;

        // units and their costs (in 128-k tiles, plus a fixed per-unit overhead
        // for the reduction and the synchronization around it)
        const int rpu = 1;  // scheduling unit: one rowblock, for every M
        std::vector<WorkItem> items((size_t)count);
        int64_t total_units = 0, total_cost = 0;
        for (int32_t i = 0; i < count; ++i) {
            const qg_gemv_desc &d = descs[i];
            WorkItem &w = items[(size_t)i];
            w = WorkItem{};
            w.packed = reinterpret_cast<const uint8_t *>(d.packed);
            w.x = d.x;
            w.y = d.y;
            w.N = (int32_t)d.N;
            w.K = (int32_t)d.K;
            w.P = (int32_t)ceil_div(d.K, aff.bits ? AFF_TILE_K : q8row ? Q8R_TILE_K : Q4_TILE_K);
            w.units = (int32_t)ceil_div(ceil_div(d.N, RB), rpu);
            w.out_f32 = out_dtype == QG_OUT_F32 ? 1 : 0;
            total_units += w.units;
            total_cost += (int64_t)w.units * ((int64_t)w.P * rpu + 2);
        }
        const int per_cu = aff.bits ? (M == 1 ? affine_gemv_wgs_per_cu() : affine_skinny_wgs_per_cu())
                           : q8row                    ? q8row_gemv_wgs_per_cu()
                           : kernel == QG_KERNEL_VALU ? q4_gemv_list_wgs_per_cu(M)
                                                      : q4_skinny_stream_wgs_per_cu();
        int64_t grid = (int64_t)cus * per_cu;
        if (grid > WL_GRID_MAX) grid = WL_GRID_MAX;
        if (grid > total_units) grid = total_units;

        // contiguous, cost-balanced ranges: workgroup j starts at the first
        // unit whose preceding cost reaches j * total / grid
        std::vector<WorkStart> starts((size_t)grid + 1);
        {
            int64_t j = 0, before = 0;
            for (int32_t i = 0; i < count && j < grid; ++i) {
                const int64_t c = (int64_t)items[(size_t)i].P * rpu + 2;
                for (int32_t u = 0; u < items[(size_t)i].units && j < grid; ++u) {
                    while (j < grid && before >= (j * total_cost) / grid) {
                        starts[(size_t)j] = WorkStart{i, u};
                        ++j;
                    }
                    before += c;
                }
            }
            for (; j <= grid; ++j) starts[(size_t)j] = WorkStart{count, 0};
        }

        // header + items + starts, uploaded through kernel arguments
        std::vector<uint32_t> words(qg_batch_worklist_bytes(count) / 4, 0u);
        uint32_t *hdr = words.data();
        hdr[0] = WL_MAGIC;
        hdr[1] = (uint32_t)count;
        hdr[2] = (uint32_t)grid;
        hdr[3] = (uint32_t)M;
        std::memcpy(words.data() + WL_HEADER_BYTES / 4, items.data(), sizeof(WorkItem) * items.size());
        const size_t starts_off = (WL_HEADER_BYTES + sizeof(WorkItem) * items.size()) / 4;
        std::memcpy(words.data() + starts_off, starts.data(), sizeof(WorkStart) * starts.size());
        const size_t nwords = starts_off + sizeof(WorkStart) * starts.size() / 4;
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        st = hip_status(launch_write_words(words.data(), nwords, reinterpret_cast<uint32_t *>(worklist), s));
        if (st != QG_OK) return st;

        plan->fmt = fmt;
        plan->M = (int32_t)M;
        plan->count = count;
        plan->out_dtype = out_dtype;
        plan->grid = (int32_t)grid;
        plan->kmax = (int32_t)kmax;
        plan->kernel = kernel;
        plan->reserved1 = 0;
        plan->worklist = worklist;
        plan->worklist_bytes = worklist_bytes;
        return QG_OK;
    } catch (...) {
        return QG_EINTERNAL;
    }
}

int qg_batch_run(const qg_batch_plan *plan, void *stream) {
    try {
        if (!plan || !plan->worklist || !aligned(plan->worklist, 16)) return QG_EINVAL;
        const AffineFmt aff = affine_decode(plan->fmt);
        const bool q8row = plan->fmt == QG_FMT_Q8_ROW;
        if ((plan->fmt != QG_FMT_Q4_ASYM_G64 && !aff.bits && !q8row) ||
            (q8row && (plan->M != 1 || plan->kernel != QG_KERNEL_VALU)) ||
            (aff.bits && ((plan->M == 1) != (plan->kernel == QG_KERNEL_VALU))) ||
            plan->M < 1 || plan->M > M_MAX ||
            plan->count < 1 || plan->count > 65536 || plan->grid < 1 ||
            plan->grid > WL_GRID_MAX || plan->kmax < format_group(plan->fmt) ||
            (plan->M == 1 && plan->kmax > GEMV_K_MAX) ||
            (plan->kernel != QG_KERNEL_VALU && plan->kernel != QG_KERNEL_MFMA) ||
            (plan->kernel == QG_KERNEL_VALU && plan->M > q4_gemv_rows_max()) ||
            plan->worklist_bytes < qg_batch_worklist_bytes(plan->count))
            return QG_EINVAL;
        const uint8_t *base = reinterpret_cast<const uint8_t *>(plan->worklist);
        const WorkItem *items = reinterpret_cast<const WorkItem *>(base + WL_HEADER_BYTES);
        const WorkStart *starts = reinterpret_cast<const WorkStart *>(items + plan->count);
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        if (q8row)
            return hip_status(launch_q8row_gemv_list(items, starts, plan->grid, plan->kmax, s));
        if (aff.bits && plan->M == 1)
            return hip_status(launch_affine_gemv_list(items, starts, plan->grid, plan->kmax,
                                                      aff.bits, aff.group, aff.bf16 != 0, s));
        if (aff.bits)
            return hip_status(launch_affine_skinny_list(items, starts, plan->grid, aff.bits,
                                                        aff.group, aff.bf16 != 0, plan->M, s));
        if (plan->kernel == QG_KERNEL_VALU)
            return hip_status(launch_q4_gemv_list(items, starts, plan->grid, plan->M, s));
        return hip_status(launch_q4_skinny_stream_list(items, starts, plan->grid, plan->M, s));
    } catch (...) {
        return QG_EINTERNAL;
    }
}

int qg_plain_read(const void *buf, size_t bytes, uint32_t *sink, int grid, void *stream) {
    try {
        if (!buf || !sink) return QG_EINVAL;
        if (bytes % 16 != 0 || grid < 1 || grid > 65536) return QG_ESHAPE;
        if (!aligned(buf, 16) || !aligned(sink, 4)) return QG_EALIGN;
        if (bytes == 0) return QG_OK;
        return hip_status(launch_plain_read(buf, bytes, sink, grid,
                                            reinterpret_cast<hipStream_t>(stream)));
    } catch (...) {
        return QG_EINTERNAL;
    }
}

}  // extern "C"
