"""Algorithmic byte and flop accounting for the decode GEMV family.

Batch-one decode reads every weight once per token with about one
multiply-add each, so its speed is bounded by memory bandwidth divided by the
bytes read per token (Uzu page, fange-kb.cn, section "Why batch-one decoding
is memory-bound": 153 GB/s / 5.2 GB = about 29 tok/s on a base M5; "MLX
Runner: An Inference Engine You Can Read", section "Optimized against a known
ceiling": 197 GB/s / 4.08 GB = about 48 tok/s, of which 41.0 tok/s is about
85%).  "Algorithmic bytes" are the bytes the computation has to move at
least once: the quantized weights with their scales, the activations in and
the outputs out.  Packing padding and re-reads are not counted.
"""
from __future__ import annotations

# bytes per weight: codes + per-group scale data
Q4_BYTES_PER_WEIGHT = 4.0 / 8 + 4.0 / 64      # 4-bit code, fp16 scale + fp16 bias per 64
Q8_BYTES_PER_WEIGHT = 1.0 + 2.0 / 32          # int8 code, fp16 scale per 32
MXFP4_BYTES_PER_WEIGHT = 0.5 + 1.0 / 32       # E2M1 code, E8M0 scale per 32

# MI355X published peaks
HBM_PEAK_GBS = 8000.0
BF16_DENSE_TFLOPS = 2500.0
I8_DENSE_TOPS = 5000.0
FP32_VECTOR_TFLOPS = 157.3

# Mean tokens produced per forward pass with speculative drafts, as the Uzu
# CLI reports it for a 9B model on a base M5 (Uzu page, fange-kb.cn, section
# "Run a model locally and inspect the runtime"): used only to express a
# verification pass rate as an equivalent decode rate.
MEAN_ACCEPTED_TOKENS = 8.39


def q4_gemm_bytes(M: int, N: int, K: int, out_bytes: int = 2) -> float:
    """Q4 weights once + bf16 activations in + outputs out."""
    return Q4_BYTES_PER_WEIGHT * N * K + 2.0 * M * K + float(out_bytes) * M * N


def q8_gemm_bytes(M: int, N: int, K: int, out_bytes: int = 2) -> float:
    """Q8 weights + int8 activations + fp32 row scales + outputs."""
    return Q8_BYTES_PER_WEIGHT * N * K + 1.0 * M * K + 4.0 * M + float(out_bytes) * M * N


def hadamard_quant_bytes(M: int, K: int) -> float:
    """bf16 activations + signs in, int8 codes + fp32 row scales out."""
    return 2.0 * M * K + K + 1.0 * M * K + 4.0 * M


def q8row_gemv_bytes(N: int, K: int, out_bytes: int = 2) -> float:
    """Weight-only int8 GEMV: one byte per weight, an fp32 scale per row, x in
    (bf16) and y out."""
    return 1.0 * N * K + 4.0 * N + 2.0 * K + float(out_bytes) * N


def affine_gemv_bytes(bits: int, group: int, N: int, K: int, out_bytes: int = 2) -> float:
    """Affine-family GEMV: bits/8 bytes per weight plus a 2-byte scale and a
    2-byte bias per group, x in (bf16) and y out."""
    return N * K * (bits / 8.0 + 4.0 / group) + 2.0 * K + float(out_bytes) * N


def moe_expert_bytes(H: int, F: int) -> float:
    """One MXFP4 expert: gate, up [F, H] and down [H, F]."""
    return 3.0 * H * F * MXFP4_BYTES_PER_WEIGHT


def moe_token_bytes(top_k: int, H: int, F: int, out_bytes: int = 2) -> float:
    """The selected experts' weights, x in, y out, and the fp32 SwiGLU
    activations written and read back once (the router ids and weights are
    negligible)."""
    return top_k * moe_expert_bytes(H, F) + 2.0 * H + float(out_bytes) * H + 2 * 4.0 * top_k * F


def moe_positions_bytes(distinct: float, T: int, top_k: int, H: int, F: int,
                        out_bytes: int = 2) -> float:
    """A pass of T positions through the layer: each distinct expert's weights
    once, X in, Y out, and per (position, slot) pair the fp32 SwiGLU
    activations and the fp32 partial output, each written and read once."""
    P = T * top_k
    return (distinct * moe_expert_bytes(H, F) + 2.0 * T * H + float(out_bytes) * T * H +
            2 * 4.0 * P * F + 2 * 4.0 * P * H)


def gemm_flops(M: int, N: int, K: int) -> float:
    return 2.0 * M * N * K


def decode_tok_per_s(bandwidth_gbs: float, bytes_per_token: float) -> float:
    """The bandwidth ceiling of batch-one decode: bandwidth / bytes per token."""
    return bandwidth_gbs * 1e9 / bytes_per_token


def decode_step_bytes(shapes, M: int = 1, out_bytes: int = 2) -> float:
    """Sum over the (item, name, N, K) GEMVs of one decode step."""
    return sum(q4_gemm_bytes(M, N, K, out_bytes) for _, _, N, K in shapes)
