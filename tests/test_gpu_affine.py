"""GPU parity: the affine weight family (2/3/4/5/6/8-bit codes, groups of
32/64/128, fp16 or bf16 scales and biases; "MLX Runner", section
"Architecture: one command buffer per token") through qgemv_pack and
qgemv_run, against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import quantized_weight_decode_dequant_amd as pkg
from quantized_weight_decode_dequant_amd import synth, weights, workloads
from helpers import assert_bf16_close, assert_f32_close, note, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
BITS = (2, 3, 4, 5, 6, 8)


def run(m, packed, x, out_dtype):
    fmt = pkg.affine_format(m.bits, m.group, m.bf16_scales)
    N, K = m.codes.shape
    y = pkg.qgemv_run(fmt, packed, N, K, weights.to_device(x, DEV), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return to_np(y)


def check(m, x):
    N, K = m.codes.shape
    ref = oracle.affine_gemv(m.codes, m.scales, m.biases, x, m.group, m.bf16_scales)
    packed = weights.pack_affine(m, DEV)
    fmt = pkg.affine_format(m.bits, m.group, m.bf16_scales)
    assert packed.numel() == pkg.packed_bytes(fmt, N, K)
    what = "bits=%d g=%d bf16=%d N=%d K=%d" % (m.bits, m.group, m.bf16_scales, N, K)
    assert_f32_close(run(m, packed, x, pkg.OUT_F32), ref, what=what + " f32")
    assert_bf16_close(run(m, packed, x, pkg.OUT_BF16), ref, what=what + " bf16")


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("group", (32, 64, 128))
@pytest.mark.parametrize("bf16", (False, True))
def test_affine_gemv(bits, group, bf16):
    """Every member of the family; 100 rows (ragged last rowblock), K = 1536
    (3 batches of 4 tiles)."""
    m = synth.affine_matrix(120, 100, 1536, bits, group, bf16)
    check(m, synth.activations(121, 1, 1536)[0])


# partial tiles (K = 96: three groups of 32; K = 320), one row, more than
# 32 rowblocks per workgroup, K at its maximum (2 and 3 bits at group 32 take
# the most LDS: x, its group sums and the offset-weighted sums, 80 KB)
@pytest.mark.parametrize("bits,group,N,K", [(3, 32, 40, 96), (5, 64, 17, 320), (2, 32, 1, 32),
                                            (6, 128, 3000, 256), (8, 64, 33, 24576),
                                            (4, 128, 70, 24576), (2, 32, 50, 24576),
                                            (3, 32, 20, 24576)])
def test_affine_gemv_shapes(bits, group, N, K):
    note("affine bits=%d g=%d N=%d K=%d" % (bits, group, N, K))
    m = synth.affine_matrix(122, N, K, bits, group, bits % 2 == 1)
    check(m, synth.activations(123, 1, K)[0])


@pytest.mark.parametrize("bits", BITS)
def test_affine_extreme_codes_onehot(bits):
    """Codes 0 and 2^bits - 1; a one-hot x returns scale * code + bias of the
    column, rounded once to fp32."""
    N, K, g = 32, 256, 64
    m = synth.affine_matrix(124, N, K, bits, g, False)
    m.codes[0, :] = (1 << bits) - 1
    m.codes[1, :] = 0
    m.codes[2, ::2] = (1 << bits) - 1
    packed = weights.pack_affine(m, DEV)
    for k in (0, 1, 63, 64, 255):
        x = synth.f32_to_bf16_bits(np.eye(1, K, k, dtype=np.float32)[0])
        ref = oracle.affine_gemv(m.codes, m.scales, m.biases, x, g, False)
        got = run(m, packed, x, pkg.OUT_F32)
        assert np.array_equal(got, ref.astype(np.float32)), (bits, k)


def test_affine_4bit_matches_q4_path():
    """AFFINE(4, 64, fp16) and QG_FMT_Q4_ASYM_G64 are the same weights in two
    packed layouts and kernels: both agree with the oracle on the 4096 x 4096
    workload."""
    q = synth.q4_matrix(0, 4096, 4096)
    x = synth.activations(0, 1, 4096)[0]
    words = q.codes.astype(np.uint64)
    codes = np.stack([(words >> (4 * i)) & 0xF for i in range(8)], axis=-1)
    m = synth.AffineMatrix(codes.reshape(4096, 4096).astype(np.uint8), q.scales, q.biases, 4, 64,
                           False)
    ref = oracle.q4_gemm(q.codes, q.scales, q.biases, x[None])[0]
    got = run(m, weights.pack_affine(m, DEV), x, pkg.OUT_F32)
    assert_f32_close(got, ref, what="affine 4-bit")
    y4 = to_np(pkg.qgemv_run(pkg.FMT_Q4_ASYM_G64, weights.pack_q4(q, DEV), 4096, 4096,
                             weights.to_device(x, DEV), out_dtype=pkg.OUT_F32))
    assert_f32_close(y4, ref, what="q4 path")


# ------------------------------------------------------------ skinny (M rows)
def run_skinny(m, packed, X, out_dtype):
    fmt = pkg.affine_format(m.bits, m.group, m.bf16_scales)
    N, K = m.codes.shape
    Y = pkg.qgemm_skinny_run(fmt, packed, X.shape[0], N, K, weights.to_device(X, DEV),
                             out_dtype=out_dtype)
    torch.cuda.synchronize()
    return to_np(Y)


def check_skinny(m, X):
    N, K = m.codes.shape
    ref = oracle.affine_gemm(m.codes, m.scales, m.biases, X, m.group, m.bf16_scales)
    packed = weights.pack_affine(m, DEV)
    what = "skinny bits=%d g=%d bf16=%d M=%d N=%d K=%d" % (m.bits, m.group, m.bf16_scales,
                                                          X.shape[0], N, K)
    assert_f32_close(run_skinny(m, packed, X, pkg.OUT_F32), ref, what=what + " f32")
    assert_bf16_close(run_skinny(m, packed, X, pkg.OUT_BF16).ravel(), ref.ravel(),
                      what=what + " bf16")


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("group", (32, 64, 128))
@pytest.mark.parametrize("bf16", (False, True))
@pytest.mark.parametrize("M", (16, 32))
def test_affine_skinny(bits, group, bf16, M):
    """Every member of the family at 16 and 32 rows; 100 output rows (ragged
    last rowblock), K = 1536."""
    m = synth.affine_matrix(125, 100, 1536, bits, group, bf16)
    check_skinny(m, synth.activations(126, M, 1536))


# 2 and 17 rows; K over several staged segments (12288 at 16 rows, 6144 at
# 32); a partial last tile; more rowblocks than one pass of the waves; M = 1
# (the GEMV)
@pytest.mark.parametrize("bits,group,M,N,K", [(4, 64, 2, 40, 256), (3, 32, 17, 33, 160),
                                              (2, 128, 16, 64, 12288), (8, 32, 32, 48, 6144),
                                              (5, 64, 16, 7000, 512), (6, 32, 32, 3000, 4096),
                                              (4, 32, 1, 77, 1024)])
def test_affine_skinny_shapes(bits, group, M, N, K):
    note("affine skinny bits=%d g=%d M=%d N=%d K=%d" % (bits, group, M, N, K))
    m = synth.affine_matrix(127, N, K, bits, group, bits % 2 == 0)
    check_skinny(m, synth.activations(128, M, K))


def test_affine_skinny_rows_equal_gemv_rows():
    """Row m of the skinny product equals the GEMV on X[m] to within the
    rounding of their different summation orders, and both match the oracle."""
    m = synth.affine_matrix(129, 300, 2048, 4, 64, False)
    X = synth.activations(130, 16, 2048)
    packed = weights.pack_affine(m, DEV)
    Y = run_skinny(m, packed, X, pkg.OUT_F32)
    for r in (0, 7, 15):
        assert_f32_close(run(m, packed, X[r], pkg.OUT_F32), Y[r], what="row %d" % r)


# ------------------------------------------------------------ grouped launch
BATCH_SHAPES = [(40, 192), (1, 64), (256, 4096), (33, 12288), (100, 1216), (17, 320),
                (3000, 256), (5, 96), (2, 32), (7, 384), (9, 24576)]


def _batch(seed, bits, group, bf16, shapes, out_dtype):
    """Matrices of one affine format with their own x and y, and the single
    qgemv_run output of each."""
    fmt = pkg.affine_format(bits, group, bf16)
    dt = torch.float32 if out_dtype == pkg.OUT_F32 else torch.bfloat16
    mats, xs, entries, singles = [], [], [], []
    for i, (N, K) in enumerate(shapes):
        m = synth.affine_matrix(seed, N, K, bits, group, bf16, item=i)
        x = synth.activations(seed + 1, 1, K, item=i)[0]
        p = weights.pack_affine(m, DEV)
        xd = weights.to_device(x, DEV)
        entries.append((p, N, K, xd, torch.empty(N, dtype=dt, device=DEV)))
        singles.append(pkg.qgemv_run(fmt, p, N, K, xd, out_dtype=out_dtype))
        mats.append(m)
        xs.append(x)
    return fmt, mats, xs, entries, singles


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("group", (32, 64, 128))
def test_affine_batch_mixed_shapes(bits, group):
    """One grouped launch over affine GEMVs of mixed shapes (partial tiles,
    one row, K up to 12288): each output against the oracle and bitwise
    equal to qgemv_run's (same kernel body, same order)."""
    out_dtype = pkg.OUT_BF16 if group == 64 else pkg.OUT_F32
    bf16 = bits % 2 == 0
    note("affine batch bits=%d g=%d" % (bits, group))
    shapes = [(N, K) for N, K in BATCH_SHAPES if K % group == 0]
    fmt, mats, xs, entries, singles = _batch(140 + bits, bits, group, bf16, shapes, out_dtype)
    plan = pkg.qg_batch_plan_build(fmt, 1, entries, out_dtype)
    pkg.qg_batch_run(plan)
    torch.cuda.synchronize()
    for (p, N, K, xd, y), s, m, x in zip(entries, singles, mats, xs):
        ref = oracle.affine_gemv(m.codes, m.scales, m.biases, x, group, bf16)
        what = "bits=%d g=%d N=%d K=%d" % (bits, group, N, K)
        if out_dtype == pkg.OUT_F32:
            assert_f32_close(to_np(y), ref, what=what)
        else:
            assert_bf16_close(to_np(y), ref, what=what)
        assert torch.equal(y, s), "batch differs from qgemv_run: " + what


@pytest.mark.parametrize("bits", (3, 4))
def test_affine_batch_split_items_bit_identical(bits):
    """Items with more rowblocks than the grid has workgroups times four, whose
    batches per rowblock (ceil(K / 512) = 7, 5, 3) are not a multiple of the
    four waves, so the grouped launch and qgemv_run cut them into workgroup
    ranges at different rowblocks: the outputs still agree bit for bit, and
    sampled rows match the oracle."""
    note("affine batch split items bits=%d" % bits)
    shapes = [(100, 1216), (18944, 3584), (7, 384), (6000, 2560), (4100, 1536)]
    fmt, mats, xs, entries, singles = _batch(170 + bits, bits, 64, False, shapes, pkg.OUT_F32)
    plan = pkg.qg_batch_plan_build(fmt, 1, entries, pkg.OUT_F32)
    pkg.qg_batch_run(plan)
    torch.cuda.synchronize()
    rng = np.random.default_rng(171)
    for (p, N, K, xd, y), s, m, x in zip(entries, singles, mats, xs):
        what = "bits=%d N=%d K=%d" % (bits, N, K)
        assert torch.equal(y, s), "batch differs from qgemv_run: " + what
        rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, min(N, 64), replace=False)]))
        ref = oracle.affine_gemv(m.codes[rows], m.scales[rows], m.biases[rows], x, 64, False)
        assert_f32_close(to_np(y)[rows], ref, what=what)


@pytest.mark.parametrize("bits,group,M", [(4, 64, 16), (2, 32, 2), (3, 128, 32), (8, 64, 17),
                                          (5, 32, 16), (6, 64, 32)])
def test_affine_batch_skinny_mixed_shapes(bits, group, M):
    """Affine verification products (M rows each) of mixed shapes in one
    grouped launch: ragged rowblocks, K over several staged segments, more
    rowblocks than one workgroup takes.  Every output bitwise equal to
    qgemm_skinny_run's (each rowblock adds its tiles in K order within one
    wave in both), sampled rows against the oracle."""
    note("affine batch skinny bits=%d g=%d M=%d" % (bits, group, M))
    bf16 = bits % 2 == 1
    fmt = pkg.affine_format(bits, group, bf16)
    shapes = [(N, K) for N, K in ((40, 256), (300, 4096), (33, 12288), (1000, 1280), (17, 384),
                                  (9000, 2048)) if K % group == 0]
    entries, singles, mats, Xs = [], [], [], []
    for i, (N, K) in enumerate(shapes):
        m = synth.affine_matrix(180 + bits, N, K, bits, group, bf16, item=i)
        X = synth.activations(181, M, K, item=i)
        p = weights.pack_affine(m, DEV)
        Xd = weights.to_device(X, DEV)
        entries.append((p, N, K, Xd, torch.empty((M, N), dtype=torch.bfloat16, device=DEV)))
        singles.append(pkg.qgemm_skinny_run(fmt, p, M, N, K, Xd))
        mats.append(m)
        Xs.append(X)
    plan = pkg.qg_batch_plan_build(fmt, M, entries)
    pkg.qg_batch_run(plan)
    torch.cuda.synchronize()
    rng = np.random.default_rng(182)
    for (p, N, K, Xd, Y), s, m, X in zip(entries, singles, mats, Xs):
        what = "bits=%d g=%d M=%d N=%d K=%d" % (bits, group, M, N, K)
        assert torch.equal(Y, s), "batch differs from qgemm_skinny_run: " + what
        rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, min(N, 24), replace=False)]))
        ref = oracle.affine_gemm(m.codes[rows], m.scales[rows], m.biases[rows], X, group, bf16)
        assert_bf16_close(to_np(Y)[:, rows].ravel(), ref.ravel(), what=what)


def test_affine_batch_layer_graph_replay():
    """A decoder layer's seven projections (4096 -> 4096, 1024, 1024, 4096,
    12288, 12288; 12288 -> 4096) at 3 bits in one launch, captured in a HIP
    graph: every replay, with eager work between, equals the eager launch,
    which equals qgemv_run per projection; sampled rows against the oracle."""
    note("affine batch layer graph")
    shapes = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (12288, 4096),
              (12288, 4096), (4096, 12288)]
    fmt, mats, xs, entries, singles = _batch(150, 3, 64, False, shapes, pkg.OUT_BF16)
    plan = pkg.qg_batch_plan_build(fmt, 1, entries)
    pkg.qg_batch_run(plan)
    torch.cuda.synchronize()
    eager = [e[4].clone() for e in entries]
    for e, s in zip(eager, singles):
        assert torch.equal(e, s)
    rng = np.random.default_rng(151)
    for (p, N, K, xd, y), m, x in zip(entries, mats, xs):
        rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 48, replace=False)]))
        ref = oracle.affine_gemv(m.codes[rows], m.scales[rows], m.biases[rows], x, 64, False)
        assert_bf16_close(to_np(y)[rows], ref, what="N=%d K=%d" % (N, K))
    g = workloads.capture_graph(lambda: pkg.qg_batch_run(plan))
    for rep in range(3):
        for e in entries:
            e[4].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, ref in zip(entries, eager):
            assert torch.equal(e[4], ref), "replay %d differs" % rep
        _ = torch.randn(1000, device=DEV).sum().item()  # unrelated eager work in between


def test_affine_batch_shared_input():
    """q, k and v on one x and gate, up on another: the plan points several
    products at the same activation buffer."""
    note("affine batch shared inputs")
    shapes = [(512, 2048), (128, 2048), (128, 2048), (1024, 2048), (1024, 2048)]
    bits, group = 5, 32
    fmt = pkg.affine_format(bits, group, True)
    x1 = synth.activations(160, 1, 2048, item=0)[0]
    x2 = synth.activations(160, 1, 2048, item=1)[0]
    xd1, xd2 = weights.to_device(x1, DEV), weights.to_device(x2, DEV)
    entries, mats, which = [], [], []
    for i, (N, K) in enumerate(shapes):
        m = synth.affine_matrix(161, N, K, bits, group, True, item=i)
        use2 = i >= 3
        entries.append((weights.pack_affine(m, DEV), N, K, xd2 if use2 else xd1,
                        torch.empty(N, dtype=torch.float32, device=DEV)))
        mats.append(m)
        which.append(x2 if use2 else x1)
    plan = pkg.qg_batch_plan_build(fmt, 1, entries, pkg.OUT_F32)
    pkg.qg_batch_run(plan)
    torch.cuda.synchronize()
    for (p, N, K, xd, y), m, x in zip(entries, mats, which):
        ref = oracle.affine_gemv(m.codes, m.scales, m.biases, x, group, True)
        assert_f32_close(to_np(y), ref, what="N=%d" % N)
