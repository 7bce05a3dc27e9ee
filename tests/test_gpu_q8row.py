"""GPU parity: weight-only int8 decode GEMV with one fp32 scale per row (the
int8 spine and output head of the Deltafin / Kimi K3 page), through the C
ABI, against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import quantized_weight_decode_dequant_amd as pkg
from quantized_weight_decode_dequant_amd import synth, weights
from helpers import assert_bf16_close, assert_f32_close, note, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
Q8R = pkg.FMT_Q8_ROW


def run(packed, N, K, x, out_dtype):
    y = pkg.qgemv_run(Q8R, packed, N, K, weights.to_device(x, DEV), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return to_np(y)


# ragged rowblocks and tiles (K = 32 is a quarter tile), more than 32
# rowblocks per workgroup, K at its maximum
@pytest.mark.parametrize("N,K", [(1, 32), (16, 128), (40, 288), (17, 4096), (100, 7168),
                                 (2000, 160), (33, 24576), (4096, 4096)])
def test_q8row_gemv(N, K):
    note("q8row gemv N=%d K=%d" % (N, K))
    m = synth.q8row_matrix(110, N, K)
    x = synth.activations(111, 1, K)[0]
    ref = oracle.q8row_gemv(m.codes, m.scales, x)
    packed = weights.pack_q8row(m, DEV)
    assert packed.numel() == pkg.packed_bytes(Q8R, N, K)
    assert_f32_close(run(packed, N, K, x, pkg.OUT_F32), ref, what="f32")
    assert_bf16_close(run(packed, N, K, x, pkg.OUT_BF16), ref, what="bf16")


def test_q8row_extremes_and_onehot():
    """Codes -128 and 127, large and tiny row scales; a one-hot x returns the
    dequantized column (scale * code, rounded once to fp32)."""
    N, K = 48, 256
    m = synth.q8row_matrix(112, N, K)
    m.codes[0, :] = -128
    m.codes[1, :] = 127
    m.codes[2, ::2] = -128
    m.codes[2, 1::2] = 127
    m.scales[3] = 2.0 ** 20
    m.scales[4] = 2.0 ** -30
    packed = weights.pack_q8row(m, DEV)
    for k in (0, 1, 127, 128, 255):
        x = synth.f32_to_bf16_bits(np.eye(1, K, k, dtype=np.float32)[0])
        got = run(packed, N, K, x, pkg.OUT_F32)
        exp = (m.scales * m.codes[:, k].astype(np.float32)).astype(np.float32)
        assert np.array_equal(got, exp), k
    x = synth.activations(113, 1, K)[0]
    assert_f32_close(run(packed, N, K, x, pkg.OUT_F32), oracle.q8row_gemv(m.codes, m.scales, x))


def test_q8row_lm_head_full():
    """The 4096 -> 151936 output head in int8 with row scales, codes drawn
    uniformly over the whole int8 range on the device; 3000 sampled rows
    (and the last rowblock) checked against the oracle."""
    N, K = 151936, 4096
    note("q8row lm_head %dx%d" % (K, N))
    g = torch.Generator(device=DEV)
    g.manual_seed(114)
    codes = torch.randint(-128, 128, (N, K), dtype=torch.int8, device=DEV, generator=g)
    scales = (torch.rand(N, dtype=torch.float32, device=DEV, generator=g) + 0.5) * 2.0 ** -10
    packed = pkg.qgemv_pack(Q8R, N, K, codes, scales)
    x = synth.activations(115, 1, K)[0]
    got_f = run(packed, N, K, x, pkg.OUT_F32)
    got_b = run(packed, N, K, x, pkg.OUT_BF16)
    rows = np.unique(np.concatenate([np.random.default_rng(116).integers(0, N, 3000),
                                     np.arange(N - 16, N)]))
    sel = torch.from_numpy(rows).to(DEV)
    ref = oracle.q8row_gemv(codes[sel].cpu().numpy(), scales[sel].cpu().numpy(), x)
    assert_f32_close(got_f[rows], ref, what="f32")
    assert_bf16_close(got_b[rows], ref, what="bf16")


def test_q8row_batch_mixed_shapes():
    """Weight-only int8 GEMVs of mixed shapes (ragged rowblocks and tiles, K up
    to its maximum, more rowblocks than one workgroup takes) in one grouped
    launch: every output bitwise equal to qgemv_run's, sampled rows against
    the oracle."""
    note("q8row batch mixed shapes")
    shapes = [(40, 192), (1, 64), (3000, 4096), (33, 24576), (100, 1216), (17, 320), (4096, 4096)]
    entries, singles, mats, xs = [], [], [], []
    for i, (N, K) in enumerate(shapes):
        m = synth.q8row_matrix(112, N, K, item=i)
        x = synth.activations(113, 1, K, item=i)[0]
        p = weights.pack_q8row(m, DEV)
        xd = weights.to_device(x, DEV)
        entries.append((p, N, K, xd, torch.empty(N, dtype=torch.bfloat16, device=DEV)))
        singles.append(pkg.qgemv_run(Q8R, p, N, K, xd))
        mats.append(m)
        xs.append(x)
    plan = pkg.qg_batch_plan_build(Q8R, 1, entries)
    pkg.qg_batch_run(plan)
    torch.cuda.synchronize()
    rng = np.random.default_rng(114)
    for (p, N, K, xd, y), s, m, x in zip(entries, singles, mats, xs):
        what = "N=%d K=%d" % (N, K)
        assert torch.equal(y, s), "batch differs from qgemv_run: " + what
        rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, min(N, 96), replace=False)]))
        ref = oracle.q8row_gemv(m.codes[rows], m.scales[rows], x)
        assert_bf16_close(to_np(y)[rows], ref, what=what)
