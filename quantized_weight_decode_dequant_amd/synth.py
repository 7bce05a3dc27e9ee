"""Seeded synthetic inputs for the weight-quantized decode GEMV family.

This module only draws random numbers and encodes them in the canonical
storage formats (bit patterns of fp16 / bf16 / int8 / packed nibbles).  It
holds none of the arithmetic of the method itself: no dequantization, no dot
product, no rotation, no quantization of activations.  Both the CPU oracle
(``oracle/``) and the HIP path consume exactly these arrays.

Every tensor is drawn from its own generator::

    numpy.random.default_rng(SeedSequence(seed, spawn_key=(stream, i, j)))

where ``stream`` names the tensor family (a small integer, table below), ``i``
the item (layer/projection index, expert index, ...) and ``j`` the tensor
within the item.  Any single item can therefore be regenerated on its own
(one projection of one layer, one expert of a pool) and always comes out
identical.

Canonical layouts (all row-major, "A x B" in a workload name means K_in x N_out,
stored [N, K] so each output row is contiguous along K):

* Q4 asymmetric group-64 (MLX affine form ``weight = scale * code + bias``,
  "MLX Runner: An Inference Engine You Can Read", section "Architecture: one
  command buffer per token"):
  ``codes`` uint32 [N, K/8], code of element k in bits 4*(k%8) .. 4*(k%8)+3
  (low nibble first); ``scales``/``biases`` fp16 bit patterns (uint16)
  [N, K/64].
* Q8 symmetric group-32 (Uzu's "Large" checkpoints, fange-kb page, section
  "How Uzu optimizes bytes and tokens per pass"): ``qw`` int8 [N, K],
  ``sw`` fp16 bits [N, K/32].
* MXFP4 (Deltafin page, section on compute, fused MXFP4 dequant + GEMV):
  ``codes`` uint8 [N, K/2], element 2i in the low nibble, 2i+1 in the high
  nibble; ``scales`` uint8 E8M0 [N, K/32].
* Activations: bf16 bit patterns (uint16) [M, K].
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# stream tags: one per tensor family, fixed forever (changing one changes data)
_S_Q4 = 1
_S_X = 2
_S_Q8 = 3
_S_Q8X = 4
_S_SIGNS = 5
_S_EXPERT = 6
_S_ROUTER = 7
_S_MOEX = 8
_S_Q8ROW = 9
_S_AFFINE = 10


def rng_for(seed: int, stream: int, i: int = 0, j: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(stream, i, j)))


# ---------------------------------------------------------------- encodings
def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even), return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f16_bits(a) -> np.ndarray:
    """Round to IEEE fp16 (numpy, round-to-nearest-even), return uint16 bits."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------- Q4 g64
@dataclass
class Q4Matrix:
    codes: np.ndarray   # uint32 [N, K/8]
    scales: np.ndarray  # uint16 (fp16 bits) [N, K/64]
    biases: np.ndarray  # uint16 (fp16 bits) [N, K/64]

    @property
    def N(self) -> int:
        return self.codes.shape[0]

    @property
    def K(self) -> int:
        return self.codes.shape[1] * 8


def q4_matrix(seed: int, N: int, K: int, item: int = 0) -> Q4Matrix:
    """codes ~ U{0..15} (uniform random words), scale = fp16(|N(0,0.02)| + 1e-3),
    bias = fp16(N(0, 0.01))."""
    if K % 64:
        raise ValueError("K must be a multiple of 64")
    r = rng_for(seed, _S_Q4, item, 0)
    codes = np.frombuffer(r.bytes(N * K // 2), dtype=np.uint32).reshape(N, K // 8).copy()
    r = rng_for(seed, _S_Q4, item, 1)
    scales = f16_bits(np.abs(r.standard_normal((N, K // 64))) * 0.02 + 1e-3)
    r = rng_for(seed, _S_Q4, item, 2)
    biases = f16_bits(r.standard_normal((N, K // 64)) * 0.01)
    return Q4Matrix(codes, scales, biases)


def bf16_normal(seed: int, shape, item: int = 0, stream: int = _S_X, std: float = 1.0) -> np.ndarray:
    """bf16(N(0, std)) bit patterns."""
    r = rng_for(seed, stream, item, 0)
    return f32_to_bf16_bits(r.standard_normal(shape) * std)


def activations(seed: int, M: int, K: int, item: int = 0) -> np.ndarray:
    """Activation tile X [M, K], bf16(N(0, 1))."""
    return bf16_normal(seed, (M, K), item=item)


# ---------------------------------------------------------------- Q8 g32
@dataclass
class Q8Matrix:
    qw: np.ndarray  # int8 [N, K]
    sw: np.ndarray  # uint16 fp16 bits [N, K/32]


def q8_matrix(seed: int, N: int, K: int, item: int = 0) -> Q8Matrix:
    """qw = clip(rint(N(0, 40)), -127, 127); sw = fp16(U[2^-13, 2^-10])."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    r = rng_for(seed, _S_Q8, item, 0)
    qw = np.clip(np.rint(r.standard_normal((N, K)) * 40.0), -127, 127).astype(np.int8)
    r = rng_for(seed, _S_Q8, item, 1)
    sw = f16_bits(r.uniform(2.0 ** -13, 2.0 ** -10, size=(N, K // 32)))
    return Q8Matrix(qw, sw)


@dataclass
class Q8RowMatrix:
    codes: np.ndarray   # int8 [N, K]
    scales: np.ndarray  # float32 [N], one per row


def q8row_matrix(seed: int, N: int, K: int, item: int = 0) -> Q8RowMatrix:
    """Weight-only int8 with a row scale: codes = clip(rint(N(0, 40)), -128,
    127) (the full int8 range), scales = float32(U[2^-11, 2^-9])."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    r = rng_for(seed, _S_Q8ROW, item, 0)
    codes = np.clip(np.rint(r.standard_normal((N, K)) * 40.0), -128, 127).astype(np.int8)
    r = rng_for(seed, _S_Q8ROW, item, 1)
    scales = r.uniform(2.0 ** -11, 2.0 ** -9, size=N).astype(np.float32)
    return Q8RowMatrix(codes, scales)


@dataclass
class AffineMatrix:
    codes: np.ndarray   # uint8 [N, K], one code per byte
    scales: np.ndarray  # uint16 fp16 or bf16 bits [N, K/group]
    biases: np.ndarray  # uint16, same
    bits: int
    group: int
    bf16_scales: bool


def affine_matrix(seed: int, N: int, K: int, bits: int, group: int, bf16_scales: bool = False,
                  item: int = 0) -> AffineMatrix:
    """Codes uniform over 0..2^bits - 1; scale = (|N(0, 0.02)| + 1e-3) * 15 /
    (2^bits - 1) (the 4-bit recipe, rescaled so weights keep their range);
    bias = N(0, 0.01); scales and biases rounded to fp16 or bf16."""
    if K % group:
        raise ValueError("K must be a multiple of the group")
    r = rng_for(seed, _S_AFFINE, item, 0)
    codes = r.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    r = rng_for(seed, _S_AFFINE, item, 1)
    sc = (np.abs(r.normal(0.0, 0.02, size=(N, K // group))) + 1e-3) * 15.0 / ((1 << bits) - 1)
    r = rng_for(seed, _S_AFFINE, item, 2)
    bi = r.normal(0.0, 0.01, size=(N, K // group))
    enc = f32_to_bf16_bits if bf16_scales else f16_bits
    return AffineMatrix(codes, enc(sc), enc(bi), bits, group, bf16_scales)


def q8_activations(seed: int, M: int, K: int, item: int = 0, outlier_frac: float = 0.01,
                   outlier_mul: float = 20.0) -> np.ndarray:
    """X = N(0, 1) with ``outlier_frac`` of the entries (iid) multiplied by
    ``outlier_mul`` before rounding to bf16."""
    r = rng_for(seed, _S_Q8X, item, 0)
    x = r.standard_normal((M, K))
    mask = r.random((M, K)) < outlier_frac
    x = np.where(mask, x * outlier_mul, x)
    return f32_to_bf16_bits(x)


def rotation_signs(seed: int, K: int, item: int = 0) -> np.ndarray:
    """Seeded +-1 sign flips, one per K index (int8)."""
    r = rng_for(seed, _S_SIGNS, item, 0)
    return np.where(r.integers(0, 2, size=K) == 1, 1, -1).astype(np.int8)


# ---------------------------------------------------------------- MXFP4 experts
@dataclass
class MXFP4Matrix:
    codes: np.ndarray   # uint8 [N, K/2]
    scales: np.ndarray  # uint8 E8M0 [N, K/32]


def mxfp4_matrix(seed: int, N: int, K: int, item: int = 0, which: int = 0,
                 e_lo: int = 118, e_hi: int = 128) -> MXFP4Matrix:
    """E2M1 codes uniform over the 16 codes (random bytes), E8M0 ~ U{e_lo..e_hi}."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    r = rng_for(seed, _S_EXPERT, item, 2 * which)
    codes = np.frombuffer(r.bytes(N * K // 2), dtype=np.uint8).reshape(N, K // 2).copy()
    r = rng_for(seed, _S_EXPERT, item, 2 * which + 1)
    scales = r.integers(e_lo, e_hi + 1, size=(N, K // 32)).astype(np.uint8)
    return MXFP4Matrix(codes, scales)


@dataclass
class Expert:
    gate: MXFP4Matrix  # [F, H]
    up: MXFP4Matrix    # [F, H]
    down: MXFP4Matrix  # [H, F]


def expert(seed: int, e: int, H: int, F: int) -> Expert:
    """Expert ``e`` of a pool: gate/up [F, H], down [H, F].  Each expert has
    its own generators, so one expert can be drawn without the others."""
    return Expert(mxfp4_matrix(seed, F, H, e, 0), mxfp4_matrix(seed, F, H, e, 1),
                  mxfp4_matrix(seed, H, F, e, 2))


def router(seed: int, E: int, top_k: int, item: int = 0):
    """Seeded router output for one token: logits ~ N(0,1)^E; ids = the top_k
    largest logits (ties -> lower index), in descending logit order; weights =
    softmax over the selected logits (float32).

    The router is upstream of the expert GEMV: its ids and weights are inputs
    to the hot path, drawn here like any other input."""
    r = rng_for(seed, _S_ROUTER, item, 0)
    logits = r.standard_normal(E)
    return router_from_logits(logits, top_k)


def router_from_logits(logits, top_k: int):
    logits = np.asarray(logits, dtype=np.float64)
    order = np.argsort(-logits, kind="stable")  # stable: equal logits keep index order
    ids = order[:top_k].astype(np.int32)
    sel = logits[ids]
    e = np.exp(sel - sel.max())
    w = (e / e.sum()).astype(np.float32)
    return ids, w


def moe_token(seed: int, H: int, item: int = 0) -> np.ndarray:
    """The token's hidden vector x [H], bf16(N(0, 1))."""
    return bf16_normal(seed, (H,), item=item, stream=_S_MOEX)


# ---------------------------------------------------------------- workloads
# The synthetic dense decode step: 36 layers of seven 4-bit projections plus
# an lm_head.  (name, K_in, N_out); stored [N, K].
DECODE_LAYERS = 36
DECODE_PROJECTIONS = (
    ("q", 4096, 4096),
    ("k", 4096, 1024),
    ("v", 4096, 1024),
    ("o", 4096, 4096),
    ("gate", 4096, 12288),
    ("up", 4096, 12288),
    ("down", 12288, 4096),
)
LM_HEAD = ("lm_head", 4096, 151936)


def decode_step_shapes(layers: int = DECODE_LAYERS):
    """List of (item, name, N, K) for every GEMV in one decode step."""
    out = []
    item = 0
    for layer in range(layers):
        for name, k_in, n_out in DECODE_PROJECTIONS:
            out.append((item, f"L{layer}.{name}", n_out, k_in))
            item += 1
    name, k_in, n_out = LM_HEAD
    out.append((item, name, n_out, k_in))
    return out
