"""GPU parity: randomized Hadamard-32 + per-row int8 quantization (bit-exact)
and the 8-bit symmetric group-32 skinny product (int32 group partials
bit-exact; fp32/bf16 outputs to tolerance), against the CPU oracle."""
import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
import quantized_weight_decode_dequant_amd as pkg
from quantized_weight_decode_dequant_amd import synth, weights
from helpers import assert_bf16_close, assert_f32_close, note, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
Q8 = pkg.FMT_Q8_SYM_G32


def gpu_had32(X, signs):
    M, K = X.shape
    Xq, sx = pkg.hadamard32_quant_run(weights.to_device(X, DEV), weights.to_device(signs, DEV), M, K)
    torch.cuda.synchronize()
    return Xq.cpu().numpy(), sx.cpu().numpy()


@pytest.mark.parametrize("M,K", [(1, 32), (3, 96), (2, 160), (2, 4128), (16, 4096), (16, 12288),
                                 (33, 640), (2, 24576), (2, 24672), (1, 49216)])
def test_hadamard_quant_bit_exact(M, K):
    note("hadamard quant M=%d K=%d" % (M, K))
    X = synth.q8_activations(40, M, K)
    signs = synth.rotation_signs(41, K)
    q_ref, sx_ref = oracle.had32_quant(X, signs)
    q, sx = gpu_had32(X, signs)
    assert np.array_equal(q, q_ref), np.argwhere(q != q_ref)[:5]
    assert np.array_equal(sx.view(np.uint32), sx_ref.view(np.uint32))


def _x_from_z(z_blocks, K, signs):
    """bf16 activations whose rotated block is exactly z (inverse transform)."""
    H = scipy.linalg.hadamard(32).astype(np.float64)
    x = np.zeros(K)
    for b, z in z_blocks:
        zz = np.zeros(32)
        zz[:len(z)] = z
        x[32 * b:32 * b + 32] = (H @ zz) / 32 * signs[32 * b:32 * b + 32]
    xb = synth.f32_to_bf16_bits(x)
    assert np.array_equal(synth.bf16_bits_to_f32(xb).astype(np.float64), x), "not bf16-exact"
    return xb


def test_hadamard_quant_ties_and_zero_row():
    """Rows built so that z * 127 / amax lands exactly on .5: round half to even
    must agree (127, 0.5 -> 0, 1.5 -> 2; -127, 2.5 -> 2, -3.5 -> -4), plus an
    all-zero row (codes 0, scale 0)."""
    K = 128
    signs = synth.rotation_signs(42, K)
    X = np.stack([_x_from_z([(1, [254, 1, 3])], K, signs),
                  _x_from_z([(0, [-254, 5, -7]), (3, [2, 0, 6])], K, signs),
                  np.zeros(K, dtype=np.uint16)])
    q_ref, sx_ref = oracle.had32_quant(X, signs)
    assert q_ref[0, 32:35].tolist() == [127, 0, 2]
    assert q_ref[1, 0:3].tolist() == [-127, 2, -4]
    assert not q_ref[2].any() and sx_ref[2] == 0
    q, sx = gpu_had32(X, signs)
    assert np.array_equal(q, q_ref)
    assert np.array_equal(sx.view(np.uint32), sx_ref.view(np.uint32))


def run_q8(w, Xq, sx, out_dtype):
    N, K = w.qw.shape
    M = Xq.shape[0]
    packed = weights.pack_q8(w, DEV)
    Y = pkg.qgemm_skinny_run(Q8, packed, M, N, K, weights.to_device(Xq, DEV),
                             weights.to_device(sx, DEV) if out_dtype != pkg.OUT_I32_GROUPS else None,
                             out_dtype=out_dtype)
    torch.cuda.synchronize()
    return Y


@pytest.mark.parametrize("M,N,K", [(1, 16, 32), (3, 40, 96), (16, 100, 384), (17, 33, 160),
                                   (32, 64, 4128)])
def test_q8_group_partials_bit_exact(M, N, K):
    note("q8 int32 partials M=%d N=%d K=%d" % (M, N, K))
    w = synth.q8_matrix(43, N, K)
    Xq, sx = oracle.had32_quant(synth.q8_activations(44, M, K), synth.rotation_signs(45, K))
    got = run_q8(w, Xq, sx, pkg.OUT_I32_GROUPS).cpu().numpy()
    assert np.array_equal(got, oracle.q8_group_acc(w.qw, Xq))


@pytest.mark.parametrize("M,N,K", [(1, 16, 32), (3, 40, 96), (16, 100, 384), (17, 33, 160),
                                   (32, 64, 4128), (16, 40, 4256), (5, 24, 8288), (32, 20, 8288),
                                   (16, 17, 32800)])
def test_q8_skinny_outputs(M, N, K):
    note("q8 outputs M=%d N=%d K=%d" % (M, N, K))
    w = synth.q8_matrix(46, N, K)
    Xq, sx = oracle.had32_quant(synth.q8_activations(47, M, K), synth.rotation_signs(48, K))
    ref = oracle.q8_gemm(w.qw, w.sw, Xq, sx)
    assert_f32_close(to_np(run_q8(w, Xq, sx, pkg.OUT_F32)), ref, what="f32")
    assert_bf16_close(to_np(run_q8(w, Xq, sx, pkg.OUT_BF16)), ref, what="bf16")


@pytest.mark.parametrize("N,K", [(12288, 4096), (4096, 12288)])
def test_int8_verification_workload_full(N, K):
    """The 8-bit workload at full size, M = 16 with 1% x20 outliers: GPU
    rotation+quantization then GPU int8 product, against the oracle's
    rotation+quantization and product from the same bf16 activations.
    Group partials compared exactly on every element; outputs on all."""
    note("int8 verification workload N=%d K=%d" % (N, K))
    M = 16
    w = synth.q8_matrix(50, N, K)
    X = synth.q8_activations(51, M, K)
    signs = synth.rotation_signs(52, K)
    Xq_ref, sx_ref = oracle.had32_quant(X, signs)
    Xq_d, sx_d = pkg.hadamard32_quant_run(weights.to_device(X, DEV), weights.to_device(signs, DEV),
                                          M, K)
    packed = weights.pack_q8(w, DEV)
    acc = pkg.qgemm_skinny_run(Q8, packed, M, N, K, Xq_d, None, out_dtype=pkg.OUT_I32_GROUPS)
    Y = pkg.qgemm_skinny_run(Q8, packed, M, N, K, Xq_d, sx_d, out_dtype=pkg.OUT_BF16)
    torch.cuda.synchronize()
    assert np.array_equal(Xq_d.cpu().numpy(), Xq_ref)
    assert np.array_equal(acc.cpu().numpy(), oracle.q8_group_acc(w.qw, Xq_ref))
    assert_bf16_close(to_np(Y), oracle.q8_gemm(w.qw, w.sw, Xq_ref, sx_ref), what="bf16")
