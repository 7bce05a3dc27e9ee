// C ABI of the library (declared in include/qgemv.h).  Every entry point
// validates its arguments on the host before any HIP call -- model inputs are
// checked explicitly before anything reaches the GPU and unsupported feature
// combinations return an error instead of being ignored ("MLX Runner: An
// Inference Engine You Can Read", section "Untrusted input, verified
// output") -- then enqueues its kernels on the caller's stream and returns.
#include <atomic>
#include <cmath>

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

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int format_group(int fmt) {
    switch (fmt) {
    case QG_FMT_Q4_ASYM_G64: return 64;
    case QG_FMT_Q8_SYM_G32: return 32;
    case QG_FMT_MXFP4_G32: return 32;
    default: return 0;
    }
}

size_t packed_bytes_for(int fmt, int64_t N, int64_t K) {
    switch (fmt) {
    case QG_FMT_Q4_ASYM_G64: return q4_packed_bytes(N, K);
    case QG_FMT_Q8_SYM_G32: return q8_packed_bytes(N, K);
    case QG_FMT_MXFP4_G32: return fp4_packed_bytes(N, K);
    default: return 0;
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
        if ((fmt == QG_FMT_Q4_ASYM_G64) != (biases != nullptr)) return QG_EINVAL;
        if (*packed_bytes < need) {
            *packed_bytes = need;
            return QG_ESIZE;
        }
        *packed_bytes = need;
        if (!aligned(packed, 16) || !aligned(codes, 16) || !aligned(scales, 2) ||
            (biases && !aligned(biases, 2)))
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
        default:
            return hip_status(launch_pack_fp4(reinterpret_cast<const uint8_t *>(codes),
                                              reinterpret_cast<const uint8_t *>(scales), rows, K,
                                              out, s));
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
        if (fmt == QG_FMT_Q4_ASYM_G64) return hip_status(launch_q4_gemv(p, xx, y, N, K, f32, cus, s));
        return hip_status(launch_fp4_gemv(p, xx, y, N, K, f32, cus, s));
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
        if (fmt == QG_FMT_MXFP4_G32) return QG_EUNSUPPORTED;
        if (fmt == QG_FMT_Q4_ASYM_G64 && out_dtype == QG_OUT_I32_GROUPS) return QG_EUNSUPPORTED;
        if (M < 0 || M > M_MAX) return QG_ESHAPE;
        if (!packed || !X || !Y) return QG_EINVAL;
        if (fmt == QG_FMT_Q8_SYM_G32 && out_dtype != QG_OUT_I32_GROUPS && !x_scales) return QG_EINVAL;
        if (fmt == QG_FMT_Q4_ASYM_G64 && x_scales) return QG_EINVAL;
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
        if (fmt == QG_FMT_Q4_ASYM_G64)
            return hip_status(launch_q4_skinny(p, reinterpret_cast<const uint16_t *>(X), Y, M, N,
                                               K, out_dtype == QG_OUT_F32, cus, s));
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
        if (!aligned(X, 16) || !aligned(Xq, 16) || !aligned(x_scales, 4)) return QG_EALIGN;
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

int moe_expert_gemv_run(const void *packed_gate, const void *packed_up, const void *packed_down,
                        size_t bytes_gate, size_t bytes_up, size_t bytes_down, int64_t E,
                        int64_t H, int64_t F, const void *x, int top_k,
                        const int32_t *expert_ids, const float *expert_w, void *workspace,
                        size_t workspace_bytes, void *y, int out_dtype, void *stream) {
    try {
        if (out_dtype != QG_OUT_BF16 && out_dtype != QG_OUT_F32 && out_dtype != QG_OUT_I32_GROUPS)
            return QG_EINVAL;
        if (out_dtype == QG_OUT_I32_GROUPS) return QG_EUNSUPPORTED;
        if (E < 1 || H < 32 || F < 32 || H % 32 || F % 32 || H > MOE_H_MAX || F > MOE_F_MAX ||
            E * F > N_MAX || E * H > N_MAX)
            return QG_ESHAPE;
        if (top_k < 0 || top_k > MOE_TOPK_MAX || top_k > E) return QG_ESHAPE;
        if (!packed_gate || !packed_up || !packed_down || !x || !y || !workspace) return QG_EINVAL;
        if (top_k > 0 && (!expert_ids || !expert_w)) return QG_EINVAL;
        if (bytes_gate != fp4_packed_bytes(E * F, H) || bytes_up != fp4_packed_bytes(E * F, H) ||
            bytes_down != fp4_packed_bytes(E * H, F))
            return QG_ESIZE;
        if (workspace_bytes < qg_moe_workspace_bytes(top_k, H, F)) return QG_ESIZE;
        if (!aligned(packed_gate, 16) || !aligned(packed_up, 16) || !aligned(packed_down, 16) ||
            !aligned(x, 16) || !aligned(workspace, 16) ||
            !aligned(y, out_dtype == QG_OUT_F32 ? 4 : 2) ||
            (expert_ids && !aligned(expert_ids, 4)) || (expert_w && !aligned(expert_w, 4)))
            return QG_EALIGN;
        int cus = 0;
        int st = device_cus(&cus);
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
