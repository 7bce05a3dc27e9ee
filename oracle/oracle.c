/*
 * Plain CPU oracle for the weight-quantized decode GEMV / skinny GEMM family.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * statement of what the hot path computes.  Only the test-suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it; the product
 * (the HIP library and its Python binding) never calls it and shares no code,
 * header, table or constant with it.
 *
 * Every floating-point result is computed in IEEE double with scalar loops in
 * the order the definition states, no SIMD, no BLAS, no blocking.  Inputs are
 * taken in their canonical storage formats (bit patterns of fp16, bf16, E8M0,
 * packed nibbles) and decoded here from the format definitions.
 *
 * Sources (the pages are cited by title and section):
 *  [MLXR]  "MLX Runner: An Inference Engine You Can Read" (21no.de),
 *          section "Architecture: one command buffer per token":
 *          affine group quantization, weight = scale x code + bias.
 *  [UZU]   Uzu on Apple M5 (fange-kb.cn), section "How Uzu optimizes bytes and
 *          tokens per pass": 4-bit asymmetric ("Medium") and 8-bit symmetric
 *          ("Large") checkpoints, activations quantized to 8 bits on the fly,
 *          block-diagonal randomized Hadamard of block 32 (+-1 entries and one
 *          global scale, random sign flips applied before mixing, exactly
 *          invertible).
 *  [K3]    Deltafin / Kimi K3 on a Mac (aihot.virxact.com), sections
 *          "How it works" (router picks the top-16 experts per layer, only
 *          those are read) and the compute list (fused MXFP4 dequant + GEMV:
 *          16-entry value table, e8m0 scale applied to the fp32 exponent).
 *  [OCP]   OCP Microscaling Formats (MX) v1.0: E2M1 element and E8M0 scale
 *          encodings (the pages name MXFP4/e8m0/e2m1 but print no table).
 *
 * Parity status of each function is stated in its comment; the pins live in
 * tests/test_oracle_pins.py and tests/golden/.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ formats */

/* IEEE binary16 -> double, from the field definition (1 sign, 5 exponent
 * bits with bias 15, 10 fraction bits; exponent 0 = subnormal). */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1024.0 + (double)f, e - 25);
    return sign ? -v : v;
}

/* bfloat16 -> double: bf16 is the upper 16 bits of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* E2M1 element [OCP]: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit.
 * Exponent field 0 is subnormal: 0 or 0.5.  Magnitudes 0,0.5,1,1.5,2,3,4,6. */
double oracle_e2m1(unsigned code)
{
    int sign = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -mag : mag;
}

/* E8M0 shared scale [OCP]: 2^(e - 127); 0xFF encodes NaN. */
double oracle_e8m0(unsigned e)
{
    if (e == 255)
        return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* ------------------------------------------------- 4-bit asymmetric group 64 */

/* Code of element k of row n: nibble k%8 (low nibble first) of word k/8. */
static unsigned q4_code(const uint32_t *codes, int64_t K, int64_t n, int64_t k)
{
    return (codes[n * (K / 8) + k / 8] >> (4 * (k % 8))) & 0xFu;
}

/* Dequantized weight w[n][k] = scale x code + bias, one (scale, bias) pair per
 * group of 64 consecutive k [MLXR]; the code is an unsigned integer 0..15 and
 * the bias carries the offset, which is what makes it asymmetric [UZU]. */
double oracle_q4_weight(const uint32_t *codes, const uint16_t *scales,
                        const uint16_t *biases, int64_t K, int64_t n, int64_t k)
{
    int64_t g = n * (K / 64) + k / 64;
    return oracle_f16_to_f64(scales[g]) * (double)q4_code(codes, K, n, k) +
           oracle_f16_to_f64(biases[g]);
}

/* Y[m][n] = sum_k w[n][k] * X[m][k]  for M activation rows (M = 1 is the
 * decode GEMV, M = 16/32 the draft-verification tile).  Plain definition:
 * dequantize each weight, multiply, sum in k order. */
void oracle_q4_gemm(int64_t M, int64_t N, int64_t K, const uint32_t *codes,
                    const uint16_t *scales, const uint16_t *biases,
                    const uint16_t *X, double *Y)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += oracle_q4_weight(codes, scales, biases, K, n, k) *
                       oracle_bf16_to_f64(X[m * K + k]);
            Y[m * N + n] = acc;
        }
}

/* ------------------------------------- randomized Hadamard-32 + int8 quant */

/* Entry (i, j) of the 32x32 Hadamard matrix in Sylvester order:
 * (-1)^popcount(i & j).  Entries are +-1; H H^T = 32 I [UZU]. */
int oracle_h32(int i, int j)
{
    int p = 0;
    for (int b = i & j; b; b >>= 1)
        p ^= (b & 1);
    return p ? -1 : 1;
}

/* z = H32 * (d (.) x) for every independent block of 32 consecutive k of every
 * row: the random sign flips d are applied first, then the block is mixed
 * [UZU].  The global 1/sqrt(32) that makes the map orthonormal is not applied
 * here; it is carried by the activation scale (oracle_quant_rows_int8).
 * Exact in double for bf16 inputs (each z is a signed sum of 32 bf16). */
void oracle_hadamard32(int64_t M, int64_t K, const uint16_t *X,
                       const int8_t *signs, double *Z)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t b = 0; b < K / 32; ++b)
            for (int i = 0; i < 32; ++i) {
                double acc = 0.0;
                for (int j = 0; j < 32; ++j) {
                    int64_t k = 32 * b + j;
                    acc += (double)oracle_h32(i, j) * (double)signs[k] *
                           oracle_bf16_to_f64(X[m * K + k]);
                }
                Z[m * K + 32 * b + i] = acc;
            }
}

/* Per-row symmetric int8 quantization of the rotated activations, done on the
 * fly [UZU]: amax = max_k |z|, q = clamp(rint(z * 127 / amax), -127, 127)
 * (ties to even, the default rounding mode), and the row scale
 * sx = amax / (127 * sqrt(32)) so that sx * q approximates the orthonormal
 * rotation R x = z / sqrt(32).  The decision is taken in double.
 * A row of zeros gives q = 0 and sx = 0. */
void oracle_quant_rows_int8(int64_t M, int64_t K, const double *Z, int8_t *Q,
                            float *sx)
{
    for (int64_t m = 0; m < M; ++m) {
        double amax = 0.0;
        for (int64_t k = 0; k < K; ++k)
            if (fabs(Z[m * K + k]) > amax)
                amax = fabs(Z[m * K + k]);
        if (amax == 0.0) {
            for (int64_t k = 0; k < K; ++k)
                Q[m * K + k] = 0;
            sx[m] = 0.0f;
            continue;
        }
        for (int64_t k = 0; k < K; ++k) {
            double t = rint(Z[m * K + k] * 127.0 / amax);
            if (t > 127.0)
                t = 127.0;
            if (t < -127.0)
                t = -127.0;
            Q[m * K + k] = (int8_t)t;
        }
        sx[m] = (float)(amax / (127.0 * sqrt(32.0)));
    }
}

/* Both steps: rotate then quantize.  M rows of K bf16 -> int8 + row scale. */
void oracle_had32_quant(int64_t M, int64_t K, const uint16_t *X,
                        const int8_t *signs, double *Z_scratch, int8_t *Q,
                        float *sx)
{
    oracle_hadamard32(M, K, X, signs, Z_scratch);
    oracle_quant_rows_int8(M, K, Z_scratch, Q, sx);
}

/* ------------------------------------------------- 8-bit symmetric group 32 */

/* Exact integer partial sums per weight group of 32:
 * ACC[m][n][g] = sum_{k in group g} qw[n][k] * qx[m][k]  (int8 x int8 -> int32;
 * |ACC| <= 32 * 127 * 127). */
void oracle_q8_group_acc(int64_t M, int64_t N, int64_t K, const int8_t *qw,
                         const int8_t *qx, int32_t *ACC)
{
    int64_t G = K / 32;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t g = 0; g < G; ++g) {
                int64_t acc = 0;
                for (int64_t k = 32 * g; k < 32 * g + 32; ++k)
                    acc += (int64_t)qw[n * K + k] * (int64_t)qx[m * K + k];
                ACC[(m * N + n) * G + g] = (int32_t)acc;
            }
}

/* Y[m][n] = sx[m] * sum_g sw[n][g] * ACC[m][n][g]: symmetric weights (no bias),
 * one fp16 scale per group of 32, int8 activations with one scale per row. */
void oracle_q8_gemm(int64_t M, int64_t N, int64_t K, const int8_t *qw,
                    const uint16_t *sw, const int8_t *qx, const float *sx,
                    double *Y)
{
    int64_t G = K / 32;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                int64_t part = 0;
                for (int64_t k = 32 * g; k < 32 * g + 32; ++k)
                    part += (int64_t)qw[n * K + k] * (int64_t)qx[m * K + k];
                acc += oracle_f16_to_f64(sw[n * G + g]) * (double)part;
            }
            Y[m * N + n] = (double)sx[m] * acc;
        }
}

/* ------------------------------------------------------------ MXFP4 experts */

/* Weight (n, k) of an MXFP4 matrix: E2M1 code of element k (element 2i in the
 * low nibble of byte i, 2i+1 in the high nibble) times the E8M0 scale of its
 * block of 32 [K3][OCP]. */
double oracle_mxfp4_weight(const uint8_t *codes, const uint8_t *scales,
                           int64_t K, int64_t n, int64_t k)
{
    unsigned byte = codes[n * (K / 2) + k / 2];
    unsigned c = (k % 2) ? (byte >> 4) : (byte & 0xFu);
    return oracle_e2m1(c) * oracle_e8m0(scales[n * (K / 32) + k / 32]);
}

/* y[n] = sum_k w[n][k] * x[k], x given in bf16. */
void oracle_mxfp4_gemv(int64_t N, int64_t K, const uint8_t *codes,
                       const uint8_t *scales, const uint16_t *x, double *y)
{
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += oracle_mxfp4_weight(codes, scales, K, n, k) *
                   oracle_bf16_to_f64(x[k]);
        y[n] = acc;
    }
}

/* Same, with x already in double (the SwiGLU output feeding the down
 * projection is kept at full precision, not rounded to bf16). */
void oracle_mxfp4_gemv_f64(int64_t N, int64_t K, const uint8_t *codes,
                           const uint8_t *scales, const double *x, double *y)
{
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += oracle_mxfp4_weight(codes, scales, K, n, k) * x[k];
        y[n] = acc;
    }
}

/* silu(a) = a / (1 + e^-a) */
double oracle_silu(double a)
{
    return a / (1.0 + exp(-a));
}

/* One token through the routed experts of one MoE layer [K3]: for each of the
 * top_k selected experts e_s with router weight w_s,
 *     g = Wgate[e_s] x,  u = Wup[e_s] x,  h = silu(g) * u,
 *     y += w_s * (Wdown[e_s] h).
 * Only the selected experts are read.  Experts are stored as arrays of E
 * matrices: gate/up codes [E][F][H/2] + scales [E][F][H/32], down codes
 * [E][H][F/2] + scales [E][H][F/32].  An id outside [0, E) contributes 0.
 * g, u, h are kept in double; y is returned in double. */
void oracle_moe(int64_t E, int64_t H, int64_t F, const uint8_t *gate_codes,
                const uint8_t *gate_scales, const uint8_t *up_codes,
                const uint8_t *up_scales, const uint8_t *down_codes,
                const uint8_t *down_scales, const uint16_t *x, int64_t top_k,
                const int32_t *ids, const float *w, double *g_scratch,
                double *u_scratch, double *h_scratch, double *d_scratch,
                double *y)
{
    for (int64_t n = 0; n < H; ++n)
        y[n] = 0.0;
    for (int64_t s = 0; s < top_k; ++s) {
        int64_t e = ids[s];
        if (e < 0 || e >= E)
            continue;
        oracle_mxfp4_gemv(F, H, gate_codes + e * F * (H / 2),
                          gate_scales + e * F * (H / 32), x, g_scratch);
        oracle_mxfp4_gemv(F, H, up_codes + e * F * (H / 2),
                          up_scales + e * F * (H / 32), x, u_scratch);
        for (int64_t f = 0; f < F; ++f)
            h_scratch[f] = oracle_silu(g_scratch[f]) * u_scratch[f];
        oracle_mxfp4_gemv_f64(H, F, down_codes + e * H * (F / 2),
                              down_scales + e * H * (F / 32), h_scratch,
                              d_scratch);
        for (int64_t n = 0; n < H; ++n)
            y[n] += (double)w[s] * d_scratch[n];
    }
}

/* ------------------------------------------------------------ int8, row scale */

/* Weight-only int8 with one fp32 scale per output row [K3]: the int8 code is
 * converted to a real number and multiplied by its row's scale,
 *     w[n][k] = scale[n] * q[n][k],
 * and y[n] = sum_k w[n][k] * x[k] with x given in bf16.  codes int8 [N][K],
 * scales fp32 [N]. */
void oracle_q8row_gemv(int64_t N, int64_t K, const int8_t *codes,
                       const float *scales, const uint16_t *x, double *y)
{
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double w = (double)scales[n] * (double)codes[n * K + k];
            acc += w * oracle_bf16_to_f64(x[k]);
        }
        y[n] = acc;
    }
}

/* ------------------------------------------------------------ affine family */

/* The affine family [MLXR]: unsigned codes q (one per byte here, q < 2^bits),
 * one scale and one bias per group of `group` consecutive k, both fp16
 * (bf16_scales = 0) or bf16 (1):
 *     w[n][k] = scale[n][k / group] * q[n][k] + bias[n][k / group],
 * y[n] = sum_k w[n][k] * x[k], x given in bf16. */
void oracle_affine_gemv(int64_t N, int64_t K, int64_t group, int bf16_scales,
                        const uint8_t *codes, const uint16_t *scales,
                        const uint16_t *biases, const uint16_t *x, double *y)
{
    int64_t G = K / group;
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            uint16_t sb = scales[n * G + k / group], bb = biases[n * G + k / group];
            double s = bf16_scales ? oracle_bf16_to_f64(sb) : oracle_f16_to_f64(sb);
            double b = bf16_scales ? oracle_bf16_to_f64(bb) : oracle_f16_to_f64(bb);
            double w = s * (double)codes[n * K + k] + b;
            acc += w * oracle_bf16_to_f64(x[k]);
        }
        y[n] = acc;
    }
}
