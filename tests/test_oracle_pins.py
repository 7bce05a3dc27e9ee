"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test pins the oracle to something other than itself: a hand-worked
example from tests/golden/ (each with its citation), a closed form, an
invariant, or a library routine that computes a special case.  Chosen so that
a dropped term, a wrong sign, a wrong index or a transposed operand in the
oracle fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from quantized_weight_decode_dequant_amd import synth
from conftest import golden_lines

BF16_ONE = 0x3F80


def onehot_bf16(K, k, val_bits=BF16_ONE):
    x = np.zeros(K, dtype=np.uint16)
    x[k] = val_bits
    return x


def ones_bf16(K):
    return np.full(K, BF16_ONE, dtype=np.uint16)


# ------------------------------------------------------------------ formats
def test_f16_decode_matches_numpy_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(c)) for c in codes])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    codes = np.concatenate([rng.integers(0, 65536, 4000), [0, 0x8000, 0x3F80, 0x0001, 0x7F7F]])
    codes = codes[((codes >> 7) & 0xFF) != 0xFF].astype(np.uint16)  # finite only
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_to_f64(int(c)) for c in codes])
    assert np.array_equal(got, ref)


def test_e2m1_table_golden():
    for code, val in golden_lines("e2m1_values.txt"):
        got = oracle.e2m1(int(code))
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_e8m0_matches_torch_float8_e8m0fnu():
    codes = np.arange(0, 255, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    got = np.array([oracle.e8m0(int(c)) for c in codes])
    assert np.array_equal(got, ref)
    assert math.isnan(oracle.e8m0(255))


# ------------------------------------------------------------------ Q4 g64
def _q4_golden():
    lines = list(golden_lines("q4_worked_example.txt"))
    K = int(lines[0][1])
    rows = []
    for r in range(2):
        words = np.zeros(K // 8, dtype=np.uint32)
        wl = [l for l in lines if l[0] == f"row{r}_words"][0]
        for item in wl[1:]:
            i, v = item.split(":")
            words[int(i)] = int(v, 16)
        gl = [l for l in lines if l[0] == f"row{r}_groups"][0]
        sb = [tuple(float(t) for t in g.split(",")) for g in gl[1:]]
        rows.append((words, sb))
    codes = np.stack([w for w, _ in rows])
    scales = synth.f16_bits(np.array([[s for s, _ in sb] for _, sb in rows]))
    biases = synth.f16_bits(np.array([[b for _, b in sb] for _, sb in rows]))
    cases = [l[1:] for l in lines if l[0] == "case"]
    return K, codes, scales, biases, cases


def test_q4_worked_example():
    K, codes, scales, biases, cases = _q4_golden()
    for row, kind, idx, expect in cases:
        x = ones_bf16(K) if kind == "ones" else onehot_bf16(K, int(idx))
        y = oracle.q4_gemm(codes, scales, biases, x[None])
        assert y[0, int(row)] == float(expect), (row, kind, idx)


def test_q4_closed_forms_random():
    """All-ones x: y[n] = sum_g (s_g * sum_k q + 64 b_g).  Zero codes: y[n] =
    sum_g b_g * sum_{k in g} x_k.  One-hot x = e_k: y = column k of W, which
    is s*q+b with q read from the nibble (cross-checked on two rows)."""
    N, K = 5, 192
    m = synth.q4_matrix(3, N, K)
    s = m.scales.view(np.float16).astype(np.float64)
    b = m.biases.view(np.float16).astype(np.float64)
    # nibbles via a byte view: little-endian, so byte i of the row holds
    # elements 2i (low nibble) and 2i+1 (high nibble)
    by = m.codes.view(np.uint8)
    q = np.empty((N, K), dtype=np.int64)
    q[:, 0::2] = by & 0xF
    q[:, 1::2] = by >> 4
    qsum = q.reshape(N, K // 64, 64).sum(-1)
    y = oracle.q4_gemm(m.codes, m.scales, m.biases, ones_bf16(K)[None])[0]
    assert np.allclose(y, (s * qsum + 64 * b).sum(-1), rtol=0, atol=1e-12)
    x = synth.activations(4, 1, K)
    xs = synth.bf16_bits_to_f32(x[0]).astype(np.float64).reshape(K // 64, 64).sum(-1)
    y0 = oracle.q4_gemm(np.zeros_like(m.codes), m.scales, m.biases, x)[0]
    assert np.allclose(y0, (b * xs).sum(-1), rtol=0, atol=1e-12)
    for k in (0, 63, 64, 131, K - 1):
        col = oracle.q4_gemm(m.codes, m.scales, m.biases, onehot_bf16(K, k)[None])[0]
        assert np.array_equal(col, s[:, k // 64] * q[:, k] + b[:, k // 64])


def test_q4_power_of_two_scaling_is_exact():
    N, K = 7, 128
    m = synth.q4_matrix(5, N, K)
    x = synth.activations(6, 2, K)
    y = oracle.q4_gemm(m.codes, m.scales, m.biases, x)
    x8 = (x.astype(np.uint32) + (3 << 7)).astype(np.uint16)  # exponent + 3 => x * 8
    y8 = oracle.q4_gemm(m.codes, m.scales, m.biases, x8)
    assert np.allclose(y8, 8 * y, rtol=1e-15, atol=0)


def test_q4_rows_are_independent_gemv():
    """M rows of the verification tile give the same result as M separate GEMVs."""
    m = synth.q4_matrix(7, 9, 256)
    X = synth.activations(8, 4, 256)
    Y = oracle.q4_gemm(m.codes, m.scales, m.biases, X)
    for i in range(4):
        assert np.array_equal(Y[i], oracle.q4_gemm(m.codes, m.scales, m.biases, X[i:i + 1])[0])


# ------------------------------------------------------- Hadamard + quant
def test_h32_is_sylvester_scipy():
    H = np.array([[oracle.h32(i, j) for j in range(32)] for i in range(32)])
    assert np.array_equal(H, scipy.linalg.hadamard(32))
    assert np.array_equal(H @ H.T, 32 * np.eye(32, dtype=np.int64))
    assert np.array_equal(H, H.T)


def test_hadamard_one_hot_gives_signed_column():
    """z = H (d . x): a one-hot x at j with sign d_j returns d_j * column j.
    Applying the signs after the mixing instead would give d . column j."""
    K = 64
    signs = synth.rotation_signs(11, K)
    H = scipy.linalg.hadamard(32)
    for j in (0, 5, 31, 32, 45):
        z = oracle.hadamard32(onehot_bf16(K, j)[None], signs)[0]
        expect = np.zeros(K)
        b = j // 32
        expect[32 * b:32 * b + 32] = signs[j] * H[:, j % 32]
        assert np.array_equal(z, expect), j


def test_hadamard_outlier_spreads_and_parseval():
    """A lone outlier 20 becomes 32 entries of magnitude 20 (20/sqrt(32) after the
    global scale): one outlier becomes many moderate values.  Parseval:
    |z|^2 = 32 |x|^2.  Exactly invertible: x = d . H z / 32."""
    K = 32
    signs = synth.rotation_signs(12, K)
    x = onehot_bf16(K, 7, synth.f32_to_bf16_bits(np.float32(20.0)).item())
    z = oracle.hadamard32(x[None], signs)[0]
    assert np.array_equal(np.abs(z), np.full(K, 20.0))
    X = synth.q8_activations(13, 3, 96)
    Z = oracle.hadamard32(X, synth.rotation_signs(14, 96))
    xf = synth.bf16_bits_to_f32(X).astype(np.float64)
    assert np.allclose((Z ** 2).sum(1), 32 * (xf ** 2).sum(1), rtol=1e-14)
    d = synth.rotation_signs(14, 96).astype(np.float64)
    H = scipy.linalg.hadamard(32)
    back = np.concatenate([(H @ Z[:, 32 * b:32 * b + 32].T).T for b in range(3)], 1) / 32 * d
    assert np.array_equal(back, xf)


def test_hadamard_all_plus_block():
    K = 32
    z = oracle.hadamard32(ones_bf16(K)[None], np.ones(K, dtype=np.int8))[0]
    expect = np.zeros(K)
    expect[0] = 32.0
    assert np.array_equal(z, expect)


def test_rotation_preserves_dot_products():
    """(R w) . (R x) = w . x with R = H D / sqrt(32) blockwise: the transform does
    not change what the model computes, up to rounding."""
    K = 128
    signs = synth.rotation_signs(15, K)
    w = synth.activations(16, 1, K)
    x = synth.activations(17, 1, K)
    zw = oracle.hadamard32(w, signs)[0] / math.sqrt(32)
    zx = oracle.hadamard32(x, signs)[0] / math.sqrt(32)
    wf = synth.bf16_bits_to_f32(w[0]).astype(np.float64)
    xf = synth.bf16_bits_to_f32(x[0]).astype(np.float64)
    assert abs(zw @ zx - wf @ xf) < 1e-12 * (np.abs(wf) @ np.abs(xf))


def test_quant_rows_worked_example():
    lines = {l[0]: l[1:] for l in golden_lines("quant_rows_worked_example.txt")}
    z = np.array([float(t) for t in lines["z"]])
    q, sx = oracle.quant_rows_int8(z[None])
    assert q[0].tolist() == [int(t) for t in lines["q"]]
    assert sx[0] == np.float32(float(lines["sx"][0]))


def test_quant_rows_zero_row_and_symmetry():
    z = np.zeros((2, 64))
    z[1, 3] = -5.0
    z[1, 9] = 2.5
    q, sx = oracle.quant_rows_int8(z)
    assert not q[0].any() and sx[0] == 0.0
    assert q[1, 3] == -127 and q[1, 9] == 64  # 2.5*127/5 = 63.5 -> 64 (even)
    q2, sx2 = oracle.quant_rows_int8(-z)
    assert np.array_equal(q2, -q) and np.array_equal(sx2, sx)


def test_had32_quant_composes_and_reconstructs():
    X = synth.q8_activations(18, 4, 256)
    signs = synth.rotation_signs(19, 256)
    Q, sx = oracle.had32_quant(X, signs)
    Q2, sx2 = oracle.quant_rows_int8(oracle.hadamard32(X, signs))
    assert np.array_equal(Q, Q2) and np.array_equal(sx, sx2)
    # sx * q approximates the orthonormal rotation R x to half a code step
    Z = oracle.hadamard32(X, signs) / math.sqrt(32)
    err = np.abs(sx[:, None].astype(np.float64) * Q - Z)
    assert np.all(err <= 0.5 * sx[:, None] * (1 + 1e-6))
    assert np.all(np.abs(Q).max(1) == 127)


# ------------------------------------------------------------------ Q8 g32
def _pattern(spec, K):
    kind, v = spec.split(":")
    v = int(v)
    if kind == "const":
        return np.full(K, v, dtype=np.int8)
    a = np.full(K, v, dtype=np.int8)
    a[K // 2:] = -v
    return a


def test_int8_worked_example():
    for _, qw_s, qx_s, sw, sx, acc, y in golden_lines("int8_worked_example.txt"):
        qw = _pattern(qw_s, 32)[None]
        qx = _pattern(qx_s, 32)[None]
        a = oracle.q8_group_acc(qw, qx)
        assert a[0, 0, 0] == int(acc)
        Y = oracle.q8_gemm(qw, synth.f16_bits([[float(sw)]]), qx, np.float32([float(sx)]))
        assert Y[0, 0] == float(y)


def test_q8_groups_and_transposition():
    """Group g covers k in [32g, 32g+32); row n of the weights pairs with row m
    of the activations (a one-hot activation picks a weight column)."""
    N, K = 3, 96
    w = synth.q8_matrix(20, N, K)
    for k in (0, 31, 32, 95):
        qx = np.zeros((1, K), dtype=np.int8)
        qx[0, k] = 1
        a = oracle.q8_group_acc(w.qw, qx)
        expect = np.zeros((1, N, K // 32), dtype=np.int32)
        expect[0, :, k // 32] = w.qw[:, k]
        assert np.array_equal(a, expect)
        Y = oracle.q8_gemm(w.qw, w.sw, qx, np.float32([1.0]))
        assert np.array_equal(Y[0], w.sw[:, k // 32].view(np.float16).astype(np.float64) * w.qw[:, k])


def test_q8_acc_matches_integer_matmul():
    """The group partials summed over groups equal the integer matrix product
    (numpy int64 matmul, a library routine)."""
    w = synth.q8_matrix(21, 6, 160)
    qx = np.clip(np.rint(np.random.default_rng(22).standard_normal((5, 160)) * 50), -127, 127).astype(np.int8)
    a = oracle.q8_group_acc(w.qw, qx)
    assert np.array_equal(a.sum(-1).astype(np.int64), qx.astype(np.int64) @ w.qw.astype(np.int64).T)


def test_rotated_weights_reproduce_unrotated_product():
    """Weights stored in the rotated basis, W' = R W blockwise, give W'.(R x) = W.x:
    the fp64 product of the rotated pair matches the unrotated one to rounding."""
    K, N = 64, 4
    signs = synth.rotation_signs(23, K)
    W = synth.activations(24, N, K)
    x = synth.activations(25, 1, K)
    Wr = oracle.hadamard32(W, signs) / math.sqrt(32)
    xr = oracle.hadamard32(x, signs)[0] / math.sqrt(32)
    ref = synth.bf16_bits_to_f32(W).astype(np.float64) @ synth.bf16_bits_to_f32(x[0]).astype(np.float64)
    assert np.allclose(Wr @ xr, ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ MXFP4
def test_mxfp4_worked_example():
    lines = list(golden_lines("mxfp4_worked_example.txt"))
    bytes_ = [int(t, 16) for t in lines[0][1:]]
    codes = np.zeros((1, 16), dtype=np.uint8)
    codes[0, :len(bytes_)] = bytes_
    for _, e, kind, idx, expect in lines[1:]:
        scales = np.full((1, 1), int(e), dtype=np.uint8)
        x = ones_bf16(32) if kind == "ones" else onehot_bf16(32, int(idx))
        assert oracle.mxfp4_gemv(codes, scales, x)[0] == float(expect)


def test_mxfp4_onehot_is_exact_column():
    N, K = 4, 96
    m = synth.mxfp4_matrix(30, N, K)
    table = np.array([float(v) for _, v in golden_lines("e2m1_values.txt")])
    for k in (0, 1, 33, 95):
        y = oracle.mxfp4_gemv(m.codes, m.scales, onehot_bf16(K, k))
        byte = m.codes[:, k // 2]
        c = (byte >> 4) if k % 2 else (byte & 0xF)
        expect = table[c] * np.ldexp(1.0, m.scales[:, k // 32].astype(np.int64) - 127)
        assert np.array_equal(y, expect)


def _q8row_example_codes():
    k = np.arange(32)
    row0 = k - 16
    row1 = np.where(k % 2 == 0, 1, -1) * 4 * (k + 1)
    return np.stack([row0, row1]).astype(np.int8)


def test_q8row_worked_example():
    lines = list(golden_lines("q8row_worked_example.txt"))
    scales = np.zeros(2, dtype=np.float32)
    for _, row, val in (l for l in lines if l[0] == "scale"):
        scales[int(row)] = float(val)
    codes = _q8row_example_codes()
    assert codes[1, 31] == -128 and codes[1, 30] == 124
    for _, row, kind, idx, expect in (l for l in lines if l[0] == "case"):
        if kind == "ones":
            x = ones_bf16(32)
        elif kind == "alt":
            x = synth.f32_to_bf16_bits(np.where(np.arange(32) % 2 == 0, 1.0, -1.0))
        else:
            x = onehot_bf16(32, int(idx))
        assert oracle.q8row_gemv(codes, scales, x)[int(row)] == float(expect)


def test_q8row_closed_forms():
    """One-hot x returns the dequantized column exactly; the result is linear
    in the row scale and in x; a zero code row gives zero; it equals the
    numpy product of the dequantized matrix."""
    m = synth.q8row_matrix(31, 6, 96)
    for k in (0, 17, 95):
        y = oracle.q8row_gemv(m.codes, m.scales, onehot_bf16(96, k))
        assert np.array_equal(y, m.scales.astype(np.float64) * m.codes[:, k])
    x = synth.activations(32, 1, 96)[0]
    y = oracle.q8row_gemv(m.codes, m.scales, x)
    assert np.array_equal(oracle.q8row_gemv(m.codes, 2 * m.scales, x), 2 * y)
    z = m.codes.copy()
    z[3] = 0
    assert oracle.q8row_gemv(z, m.scales, x)[3] == 0.0
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = (m.scales.astype(np.float64)[:, None] * m.codes.astype(np.float64)) @ xf
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())


def _affine_example(name):
    """(codes, scales, biases, group, bf16) of the worked example `name`."""
    k = np.arange(128)
    if name == "A":
        return ((k[:32] % 8)[None].astype(np.uint8), np.array([[0x3F00]], np.uint16),
                np.array([[0xBF80]], np.uint16), 32, True)
    if name == "B":
        c = np.zeros((1, 32), np.uint8)
        c[0, 0], c[0, 1] = 255, 128
        return c, np.array([[0x3C00]], np.uint16), np.array([[0x3E80]], np.uint16), 32, True
    if name == "C":
        c = np.where(k < 64, 3, 1)[None].astype(np.uint8)
        return (c, np.array([[0x3C00, 0x4000]], np.uint16), np.array([[0x0000, 0xB800]], np.uint16),
                64, False)
    c = (63 - (k % 64))[None].astype(np.uint8)
    return c, np.array([[0x3000]], np.uint16), np.array([[0x3C00]], np.uint16), 128, False


def test_affine_worked_examples():
    for _, name, kind, idx, expect in golden_lines("affine_worked_example.txt"):
        codes, sc, bi, g, bf = _affine_example(name)
        K = codes.shape[1]
        x = ones_bf16(K) if kind == "ones" else onehot_bf16(K, int(idx))
        assert oracle.affine_gemv(codes, sc, bi, x, g, bf)[0] == float(expect), (name, kind)


def test_affine_4bit_g64_equals_q4():
    """The affine family at 4 bits, group 64, fp16 is the Q4 format: the same
    matrix through both oracles (one code per byte against eight nibbles per
    word) gives the same result bit for bit."""
    m = synth.q4_matrix(33, 24, 256)
    x = synth.activations(34, 1, 256)
    words = m.codes.astype(np.uint64)
    codes = np.stack([(words >> (4 * i)) & 0xF for i in range(8)], axis=-1)
    codes = codes.reshape(24, 256).astype(np.uint8)
    y4 = oracle.q4_gemm(m.codes, m.scales, m.biases, x)[0]
    ya = oracle.affine_gemv(codes, m.scales, m.biases, x[0], 64, False)
    assert np.array_equal(ya, y4)


@pytest.mark.parametrize("bits,group,bf16", [(2, 32, False), (3, 128, True), (5, 64, False),
                                             (6, 32, True), (8, 128, False)])
def test_affine_closed_forms(bits, group, bf16):
    """One-hot x returns scale * code + bias of that column exactly; the
    result equals the numpy product of the dequantized matrix; codes at
    2^bits - 1 are taken whole."""
    N, K = 5, 256
    m = synth.affine_matrix(35, N, K, bits, group, bf16)
    m.codes[0, :] = (1 << bits) - 1
    dec = ((lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)) if bf16
           else (lambda b: b.view(np.float16).astype(np.float64)))
    s = np.repeat(dec(m.scales), group, axis=1)
    b = np.repeat(dec(m.biases), group, axis=1)
    W = s * m.codes + b
    for k in (0, 31, 32, 255):
        y = oracle.affine_gemv(m.codes, m.scales, m.biases, onehot_bf16(K, k), group, bf16)
        assert np.array_equal(y, W[:, k])
    x = synth.activations(36, 1, K)[0]
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y = oracle.affine_gemv(m.codes, m.scales, m.biases, x, group, bf16)
    assert np.allclose(y, W @ xf, rtol=1e-12, atol=1e-12 * np.abs(W @ xf).max())


def test_silu_matches_torch():
    a = np.linspace(-30, 30, 601)
    ref = torch.nn.functional.silu(torch.from_numpy(a)).numpy()
    got = np.array([oracle.silu(v) for v in a])
    assert np.allclose(got, ref, rtol=1e-15, atol=1e-300)
    assert oracle.silu(0.0) == 0.0


def _uniform_expert_pool(E, H, F, gate_byte, up_byte, down_byte, scale=127):
    gc = np.full((E, F, H // 2), gate_byte, dtype=np.uint8)
    uc = np.full((E, F, H // 2), up_byte, dtype=np.uint8)
    dc = np.full((E, H, F // 2), down_byte, dtype=np.uint8)
    gs = np.full((E, F, H // 32), scale, dtype=np.uint8)
    us = gs.copy()
    ds = np.full((E, H, F // 32), scale, dtype=np.uint8)
    return gc, gs, uc, us, dc, ds


def test_moe_closed_form_chain():
    """Expert 1: gate weights all 1.0, up all 0.5, down all 1.0 (E8M0 127);
    x = ones (H = 32).  g = 32, u = 16, h = silu(32) * 16 = 512 / (1 + e^-32),
    down row = F * h.  With one expert of weight 0.25:
    y = 0.25 * 32 * 512 / (1 + e^-32).  Expert 0 holds other values, so
    reading the wrong expert fails.  (silu on u instead of g, or gate and up
    swapped, would give a different value.)"""
    E, H, F = 2, 32, 32
    gc, gs, uc, us, dc, ds = _uniform_expert_pool(E, H, F, 0x22, 0x11, 0x22)
    gc[0] = 0x77
    uc[0] = 0x77
    y = oracle.moe(gc, gs, uc, us, dc, ds, ones_bf16(H), np.array([1], np.int32),
                   np.float32([0.25]))
    expect = 0.25 * F * 512.0 / (1.0 + math.exp(-32.0))
    assert np.allclose(y, expect, rtol=1e-15, atol=0)


def test_moe_invariants():
    E, H, F, top_k = 6, 64, 96, 3
    ex = [synth.expert(40, e, H, F) for e in range(E)]
    gc = np.stack([e.gate.codes for e in ex])
    gs = np.stack([e.gate.scales for e in ex])
    uc = np.stack([e.up.codes for e in ex])
    us = np.stack([e.up.scales for e in ex])
    dc = np.stack([e.down.codes for e in ex])
    ds = np.stack([e.down.scales for e in ex])
    x = synth.moe_token(41, H)
    ids, w = synth.router(42, E, top_k)
    y = oracle.moe(gc, gs, uc, us, dc, ds, x, ids, w)
    # permutation of the (id, weight) pairs
    p = np.array([2, 0, 1])
    assert np.allclose(oracle.moe(gc, gs, uc, us, dc, ds, x, ids[p], w[p]), y, rtol=1e-12, atol=1e-12)
    # linear in the router weights
    y2 = oracle.moe(gc, gs, uc, us, dc, ds, x, ids, (2 * w).astype(np.float32))
    assert np.allclose(y2, 2 * y, rtol=1e-14, atol=0)
    # the sum over experts equals the per-expert chain (top_k = 1 each)
    acc = sum(oracle.moe(gc, gs, uc, us, dc, ds, x, ids[s:s + 1], w[s:s + 1]) for s in range(top_k))
    assert np.allclose(acc, y, rtol=1e-12, atol=1e-12)
    # top_k = 1, w = 1: plain gate/up/SwiGLU/down chain of one expert
    e = int(ids[0])
    g = oracle.mxfp4_gemv(gc[e], gs[e], x)
    u = oracle.mxfp4_gemv(uc[e], us[e], x)
    h = g / (1 + np.exp(-g)) * u
    d = oracle.mxfp4_gemv(dc[e], ds[e], h)
    y1 = oracle.moe(gc, gs, uc, us, dc, ds, x, ids[:1], np.float32([1.0]))
    assert np.allclose(y1, d, rtol=1e-13, atol=1e-13)
    # up weights all zero -> y = 0 exactly
    y0 = oracle.moe(gc, gs, np.zeros_like(uc), us, dc, ds, x, ids, w)
    assert not np.any(y0)
    # an out-of-range id contributes nothing
    bad = ids.copy()
    bad[1] = E + 5
    keep = oracle.moe(gc, gs, uc, us, dc, ds, x, ids[[0, 2]], w[[0, 2]])
    assert np.array_equal(oracle.moe(gc, gs, uc, us, dc, ds, x, bad, w), keep)


def _dequant_mxfp4_numpy(codes, scales, table):
    """[N, K] float64 from the E2M1 table (golden file) and 2^(e - 127)."""
    lo = codes & 0xF
    hi = codes >> 4
    c = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)
    s = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return table[c] * np.repeat(s, 32, axis=1)


def test_moe_positions_brute_force():
    """T positions through the routed experts, against a brute-force numpy
    evaluation (golden E2M1 table, float64 matmuls): position 1 and 3 share
    expert 2, position 2 repeats an expert within its slots and position 3
    has an out-of-range id.  Also: reordering the positions reorders the
    rows exactly."""
    E, H, F = 5, 64, 96
    ex = [synth.expert(43, e, H, F) for e in range(E)]
    pool = tuple(np.stack([f(e) for e in ex]) for f in (
        lambda e: e.gate.codes, lambda e: e.gate.scales, lambda e: e.up.codes,
        lambda e: e.up.scales, lambda e: e.down.codes, lambda e: e.down.scales))
    X = np.stack([synth.moe_token(44, H, item=t) for t in range(4)])
    ids = np.array([[0, 4], [2, 1], [3, 3], [2, E + 1]], dtype=np.int32)
    w = np.array([[0.75, 0.25], [0.5, 0.5], [0.4, 0.6], [1.0, 0.3]], dtype=np.float32)
    Y = oracle.moe_positions(*pool, X, ids, w)
    table = np.array([float(v) for _, v in golden_lines("e2m1_values.txt")])
    xf = (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    gc, gs, uc, us, dc, ds = pool
    for t in range(4):
        ref = np.zeros(H)
        for s in range(2):
            e = int(ids[t, s])
            if not 0 <= e < E:
                continue
            g = _dequant_mxfp4_numpy(gc[e], gs[e], table) @ xf[t]
            u = _dequant_mxfp4_numpy(uc[e], us[e], table) @ xf[t]
            h = g / (1.0 + np.exp(-g)) * u
            ref += float(w[t, s]) * (_dequant_mxfp4_numpy(dc[e], ds[e], table) @ h)
        assert np.allclose(Y[t], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    perm = np.array([3, 1, 0, 2])
    assert np.array_equal(oracle.moe_positions(*pool, X[perm], ids[perm], w[perm]), Y[perm])


def test_router_equal_logits_and_ties():
    ids, w = synth.router_from_logits(np.zeros(384), 16)
    assert ids.tolist() == list(range(16))
    assert np.allclose(w, 1 / 16)
    ids, w = synth.router(0, 384, 16)
    assert len(set(ids.tolist())) == 16 and abs(float(w.sum()) - 1) < 1e-6
