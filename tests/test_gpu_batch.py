"""GPU parity of the grouped launch (qg_batch_plan_build + qg_batch_run):
many independent 4-bit GEMVs / skinny products in one kernel, against the
oracle, bitwise against the single-matrix entry points (same arithmetic in
the same order), and under HIP-graph replay."""
import numpy as np
import pytest
import torch

import oracle
import quantized_weight_decode_dequant_amd as pkg
from quantized_weight_decode_dequant_amd import synth, weights, workloads
from helpers import assert_bf16_close, assert_f32_close, assert_same, note, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
Q4 = pkg.FMT_Q4_ASYM_G64

SHAPES = [(40, 192), (1, 64), (256, 4096), (33, 12288), (100, 1216), (1024, 4096), (17, 320)]


def _mats(seed, shapes):
    return [synth.q4_matrix(seed, N, K, item=i) for i, (N, K) in enumerate(shapes)]


@pytest.mark.parametrize("out_dtype", [pkg.OUT_F32, pkg.OUT_BF16])
def test_batch_m1_mixed_shapes(out_dtype):
    note("batch M=1 mixed shapes out=%d" % out_dtype)
    mats = _mats(90, SHAPES)
    xs = [synth.activations(91, 1, m.K, item=i) for i, m in enumerate(mats)]
    dt = torch.float32 if out_dtype == pkg.OUT_F32 else torch.bfloat16
    entries, singles = [], []
    for m, x in zip(mats, xs):
        p = weights.pack_q4(m, DEV)
        xd = weights.to_device(x[0], DEV)
        y = torch.empty(m.N, dtype=dt, device=DEV)
        entries.append((p, m.N, m.K, xd, y))
        singles.append(pkg.qgemv_run(Q4, p, m.N, m.K, xd, out_dtype=out_dtype))
    plan = pkg.qg_batch_plan_build(Q4, 1, entries, out_dtype)
    pkg.qg_batch_run(plan)
    torch.cuda.synchronize()
    for (p, N, K, xd, y), s, m, x in zip(entries, singles, mats, xs):
        ref = oracle.q4_gemm(m.codes, m.scales, m.biases, x)[0]
        got = to_np(y)
        if out_dtype == pkg.OUT_F32:
            assert_f32_close(got, ref, what="N=%d K=%d" % (N, K))
        else:
            assert_bf16_close(got, ref, what="N=%d K=%d" % (N, K))
        assert_same(y, s, "batch vs qgemv_run N=%d K=%d" % (N, K))


@pytest.mark.parametrize("M", [2, 3, 4, 5, 16, 17, 32])
def test_batch_skinny_mixed_shapes(M):
    note("batch skinny M=%d" % M)
    shapes = [(40, 192), (256, 4096), (33, 1216), (130, 640), (48, 12288), (300, 8256)]
    mats = _mats(92, shapes)
    Xs = [synth.activations(93, M, m.K, item=i) for i, m in enumerate(mats)]
    entries, singles = [], []
    for m, X in zip(mats, Xs):
        p = weights.pack_q4(m, DEV)
        Xd = weights.to_device(X, DEV)
        Y = torch.empty((M, m.N), dtype=torch.float32, device=DEV)
        entries.append((p, m.N, m.K, Xd, Y))
        singles.append(pkg.qgemm_skinny_run(Q4, p, M, m.N, m.K, Xd, out_dtype=pkg.OUT_F32))
    plan = pkg.qg_batch_plan_build(Q4, M, entries, pkg.OUT_F32)
    pkg.qg_batch_run(plan)
    torch.cuda.synchronize()
    for (p, N, K, Xd, Y), s, m, X in zip(entries, singles, mats, Xs):
        # the grouped launch streams every rowblock through one wave; a single
        # matrix this small splits each rowblock's K over the waves instead, so
        # the two round differently: both are checked against the oracle
        ref = oracle.q4_gemm(m.codes, m.scales, m.biases, X)
        assert_f32_close(to_np(Y), ref, what="batch N=%d K=%d" % (N, K))
        assert_f32_close(to_np(s), ref, what="single N=%d K=%d" % (N, K))


def test_batch_graph_replay():
    """The grouped launch captured in a HIP graph: several replays, with eager
    work and synchronizations between them, each checked against the eager
    result."""
    note("batch graph replay")
    mats = _mats(94, [(256, 4096), (1024, 4096), (64, 12288)])
    entries = []
    for i, m in enumerate(mats):
        p = weights.pack_q4(m, DEV)
        x = weights.to_device(synth.activations(95, 1, m.K, item=i)[0], DEV)
        entries.append((p, m.N, m.K, x, torch.empty(m.N, dtype=torch.bfloat16, device=DEV)))
    plan = pkg.qg_batch_plan_build(Q4, 1, entries)
    pkg.qg_batch_run(plan)
    torch.cuda.synchronize()
    eager = [e[4].clone() for e in entries]
    g = workloads.capture_graph(lambda: pkg.qg_batch_run(plan))
    for rep in range(4):
        for e in entries:
            e[4].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, ref in zip(entries, eager):
            assert_same(e[4], ref, "replay %d" % rep)
        _ = torch.randn(1000, device=DEV).sum().item()  # unrelated eager work in between


def test_batch_decode_step_full():
    """The whole synthetic decode step (253 GEMVs, 4.26 GB) in one launch:
    every output bitwise equal to qgemv_run's, and sampled rows of every
    projection kind against the oracle."""
    note("batch decode step full")
    step = workloads.build_decode_step(0)
    plan = pkg.qg_batch_plan_build(Q4, 1, [(g.packed, g.N, g.K, g.x, g.y) for g in step.gemvs])
    pkg.qg_batch_run(plan)
    torch.cuda.synchronize()
    got = [g.y.clone() for g in step.gemvs]
    workloads.run_step_eager(step)
    torch.cuda.synchronize()
    for g, b in zip(step.gemvs, got):
        assert_same(b, g.y, "grouped vs qgemv_run " + g.name)
    rng = np.random.default_rng(96)
    # every projection kind of the first layer (q, k, v, o, gate, up, down),
    # one of the last layer and the lm_head
    for idx in (0, 1, 2, 3, 4, 5, 6, 250, 252):
        item, name, N, K = synth.decode_step_shapes()[idx]
        m = synth.q4_matrix(0, N, K, item=item)
        x = synth.activations(0, 1, K, item=item)
        rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 64, replace=False)]))
        ref = oracle.q4_gemm(m.codes[rows], m.scales[rows], m.biases[rows], x)[0]
        assert_bf16_close(to_np(got[idx])[rows], ref, what=name)


@pytest.mark.parametrize("M,kernel", [(4, pkg.KERNEL_VALU), (4, pkg.KERNEL_AUTO),
                                      (16, pkg.KERNEL_AUTO), (32, pkg.KERNEL_AUTO)])
def test_batch_verification_pass_full(M, kernel):
    """The whole verification pass (every projection of the decode step against
    its own M-row activation tile) in one launch: sampled output columns of
    several projections against the oracle, and (default kernel) the lm_head
    output bitwise equal to a single-matrix qgemm_skinny_run."""
    note("batch verification pass M=%d kernel=%d" % (M, kernel))
    step = workloads.build_decode_step(0, skinny_m=M)
    plan = pkg.qg_batch_plan_build(Q4, M, [(g.packed, g.N, g.K, g.X, g.Y) for g in step.gemvs],
                                   kernel=kernel)
    pkg.qg_batch_run(plan)
    torch.cuda.synchronize()
    rng = np.random.default_rng(97)
    for idx in (0, 1, 2, 3, 4, 5, 6, 251, 252):
        item, name, N, K = synth.decode_step_shapes()[idx]
        m = synth.q4_matrix(0, N, K, item=item)
        X = synth.activations(1, M, K, item=item)
        rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 48, replace=False)]))
        ref = oracle.q4_gemm(m.codes[rows], m.scales[rows], m.biases[rows], X)
        assert_bf16_close(to_np(step.gemvs[idx].Y)[:, rows], ref, what="%s M=%d" % (name, M))
    if kernel == pkg.KERNEL_AUTO:
        g = step.gemvs[-1]
        single = pkg.qgemm_skinny_run(Q4, g.packed, M, g.N, g.K, g.X)
        torch.cuda.synchronize()
        assert_same(g.Y, single, "grouped vs single " + g.name)


@pytest.mark.parametrize("M,kernel", [(2, pkg.KERNEL_AUTO), (3, pkg.KERNEL_AUTO),
                                      (5, pkg.KERNEL_AUTO), (17, pkg.KERNEL_AUTO),
                                      (3, pkg.KERNEL_VALU), (1, pkg.KERNEL_MFMA)])
@pytest.mark.parametrize("out_dtype", [pkg.OUT_F32, pkg.OUT_BF16])
def test_batch_skinny_writes_stay_inside_y(M, kernel, out_dtype):
    """Every output tile lives inside a larger buffer filled with a sentinel:
    after the grouped launch the bytes past each Y (ragged N, M not a multiple
    of 16) are unchanged and Y matches the oracle."""
    note("batch skinny bounds M=%d kernel=%d out=%d" % (M, kernel, out_dtype))
    shapes = [(40, 192), (33, 1216), (130, 640)]
    mats = _mats(98, shapes)
    dt = torch.float32 if out_dtype == pkg.OUT_F32 else torch.bfloat16
    pad = 4096
    entries, bufs = [], []
    for i, m in enumerate(mats):
        p = weights.pack_q4(m, DEV)
        Xd = weights.to_device(synth.activations(99, M, m.K, item=i), DEV)
        buf = torch.full((M * m.N + pad,), 7.0, dtype=dt, device=DEV)
        Y = buf[:M * m.N].view(M, m.N)
        entries.append((p, m.N, m.K, Xd, Y))
        bufs.append(buf)
    plan = pkg.qg_batch_plan_build(Q4, M, entries, out_dtype, kernel=kernel)
    pkg.qg_batch_run(plan)
    torch.cuda.synchronize()
    check = assert_f32_close if out_dtype == pkg.OUT_F32 else assert_bf16_close
    for i, ((p, N, K, Xd, Y), buf, m) in enumerate(zip(entries, bufs, mats)):
        assert torch.all(buf[M * N:] == 7.0), "write past Y for N=%d K=%d" % (N, K)
        ref = oracle.q4_gemm(m.codes, m.scales, m.biases, synth.activations(99, M, m.K, item=i))
        check(to_np(Y), ref, what="N=%d K=%d" % (N, K))


@pytest.mark.parametrize("M", [2, 16, 17, 32])
@pytest.mark.parametrize("out_dtype", [pkg.OUT_F32, pkg.OUT_BF16])
def test_single_skinny_writes_stay_inside_y(M, out_dtype):
    """The same sentinel check for single-matrix calls (the K-split kernel for
    small matrices)."""
    note("single skinny bounds M=%d out=%d" % (M, out_dtype))
    dt = torch.float32 if out_dtype == pkg.OUT_F32 else torch.bfloat16
    check = assert_f32_close if out_dtype == pkg.OUT_F32 else assert_bf16_close
    for i, m in enumerate(_mats(102, [(40, 192), (33, 2112), (130, 4160)])):
        X = synth.activations(103, M, m.K, item=i)
        buf = torch.full((M * m.N + 4096,), 7.0, dtype=dt, device=DEV)
        Y = buf[:M * m.N].view(M, m.N)
        pkg.qgemm_skinny_run(Q4, weights.pack_q4(m, DEV), M, m.N, m.K, weights.to_device(X, DEV),
                             Y=Y, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.all(buf[M * m.N:] == 7.0), "write past Y for N=%d K=%d" % (m.N, m.K)
        check(to_np(Y), oracle.q4_gemm(m.codes, m.scales, m.biases, X), what="N=%d K=%d" % (m.N, m.K))


@pytest.mark.parametrize("M,kernel", [(1, pkg.KERNEL_VALU), (2, pkg.KERNEL_VALU),
                                      (3, pkg.KERNEL_VALU), (4, pkg.KERNEL_VALU),
                                      (1, pkg.KERNEL_MFMA), (2, pkg.KERNEL_MFMA)])
def test_batch_forced_kernel(M, kernel):
    """Either kernel family forced on a mixed list (ragged N, K spanning
    several staged segments of both kernels) agrees with the oracle; the VALU
    family at M = 1 is the default kernel, bit for bit."""
    note("batch forced kernel M=%d kernel=%d" % (M, kernel))
    shapes = [(40, 192), (256, 4096), (33, 1216), (130, 640), (48, 12288), (70, 3136)]
    mats = _mats(100, shapes)
    Xs = [synth.activations(101, M, m.K, item=i) for i, m in enumerate(mats)]
    entries = []
    for m, X in zip(mats, Xs):
        Xd = weights.to_device(X, DEV)
        entries.append((weights.pack_q4(m, DEV), m.N, m.K, Xd,
                        torch.empty((M, m.N), dtype=torch.float32, device=DEV)))
    plan = pkg.qg_batch_plan_build(Q4, M, entries, pkg.OUT_F32, kernel=kernel)
    assert plan.plan.kernel == kernel
    pkg.qg_batch_run(plan)
    torch.cuda.synchronize()
    for (p, N, K, Xd, Y), m, X in zip(entries, mats, Xs):
        assert_f32_close(to_np(Y), oracle.q4_gemm(m.codes, m.scales, m.biases, X),
                         what="N=%d K=%d" % (N, K))
    if M == 1 and kernel == pkg.KERNEL_VALU:
        auto = [(p, N, K, Xd, torch.empty_like(Y)) for p, N, K, Xd, Y in entries]
        plan_a = pkg.qg_batch_plan_build(Q4, 1, auto, pkg.OUT_F32)
        assert plan_a.plan.kernel == pkg.KERNEL_VALU
        pkg.qg_batch_run(plan_a)
        torch.cuda.synchronize()
        for e, a in zip(entries, auto):
            assert_same(e[4], a[4], "repeat")


@pytest.mark.parametrize("M", [1, 16])
def test_batch_shared_inputs(M):
    """One layer's projections with shared inputs in one launch: q, k and v
    read the same x, gate and up the same x (the fused form of a layer's
    input projections); each output equals its own single call bit for bit
    and the oracle."""
    note("batch shared inputs M=%d" % M)
    H, Hk, F = 1024, 256, 2048
    shapes = [("q", H, H), ("k", Hk, H), ("v", Hk, H), ("gate", F, H), ("up", F, H)]
    mats = [synth.q4_matrix(138, N, K, item=i) for i, (_, N, K) in enumerate(shapes)]
    xa = synth.activations(139, M, H, item=0)
    xb = synth.activations(139, M, H, item=1)
    xa_d = weights.to_device(xa if M > 1 else xa[0], DEV)
    xb_d = weights.to_device(xb if M > 1 else xb[0], DEV)
    entries, refs = [], []
    for (name, N, K), m in zip(shapes, mats):
        shared = xa_d if name in ("q", "k", "v") else xb_d
        y = torch.empty((M, N) if M > 1 else (N,), dtype=torch.float32, device=DEV)
        entries.append((weights.pack_q4(m, DEV), N, K, shared, y))
        refs.append(oracle.q4_gemm(m.codes, m.scales, m.biases, xa if name in ("q", "k", "v") else xb))
    plan = pkg.qg_batch_plan_build(Q4, M, entries, pkg.OUT_F32)
    pkg.qg_batch_run(plan)
    torch.cuda.synchronize()
    for (p, N, K, x, y), ref in zip(entries, refs):
        got = to_np(y).reshape(M, N)
        assert_f32_close(got, ref, what="shared-input product N=%d" % N)
        if M == 1:
            single = pkg.qgemv_run(Q4, p, N, K, x, out_dtype=pkg.OUT_F32)
        else:
            single = pkg.qgemm_skinny_run(Q4, p, M, N, K, x, out_dtype=pkg.OUT_F32)
        torch.cuda.synchronize()
        if M == 1:
            assert_same(y, single, "grouped vs single")
