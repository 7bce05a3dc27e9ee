"""GPU parity: MXFP4 decode GEMV and the routed-expert MoE layer for one
token (gather by device-resident router ids, gate/up, SwiGLU, down, weighted
combine), against the CPU oracle."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import quantized_weight_decode_dequant_amd as pkg
from quantized_weight_decode_dequant_amd import synth, weights
from helpers import assert_bf16_close, assert_f32_close, note, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
FP4 = pkg.FMT_MXFP4_G32


def gemv_fp4(m, x, out_dtype):
    N, K = m.codes.shape[0], m.codes.shape[1] * 2
    packed = weights.pack_mxfp4(m.codes, m.scales, DEV)
    y = pkg.qgemv_run(FP4, packed, N, K, weights.to_device(x, DEV), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return to_np(y)


@pytest.mark.parametrize("N,K", [(1, 32), (40, 288), (100, 7168), (64, 2048), (17, 24576)])
def test_mxfp4_gemv(N, K):
    note("mxfp4 gemv N=%d K=%d" % (N, K))
    m = synth.mxfp4_matrix(60, N, K)
    x = synth.moe_token(61, K)
    ref = oracle.mxfp4_gemv(m.codes, m.scales, x)
    assert_f32_close(gemv_fp4(m, x, pkg.OUT_F32), ref, what="f32")
    assert_bf16_close(gemv_fp4(m, x, pkg.OUT_BF16), ref, what="bf16")


def test_mxfp4_gemv_onehot_is_exact():
    """E2M1 * 2^(e-127) * 1.0 is exact in fp32, so a one-hot x returns the
    dequantized column bit-exactly."""
    m = synth.mxfp4_matrix(62, 48, 512)
    for k in (0, 1, 255, 256, 511):
        x = synth.f32_to_bf16_bits(np.eye(1, 512, k, dtype=np.float32)[0])
        assert np.array_equal(gemv_fp4(m, x, pkg.OUT_F32), oracle.mxfp4_gemv(m.codes, m.scales, x))


@pytest.mark.parametrize("e8m0", (1, 252))
def test_mxfp4_gemv_scale_extremes(e8m0):
    """Every block scaled by the smallest (2^-126) or the largest (2^125)
    E8M0 scale the library supports (above 252, +-6 times the scale
    overflows bf16 and fp32): a one-hot x returns the dequantized column
    bit-exactly (at 2^-126 the half-valued codes give the fp32 subnormal
    2^-127), and a random x matches the oracle."""
    note("mxfp4 gemv e8m0=%d" % e8m0)
    N, K = 48, 512
    m = synth.mxfp4_matrix(63, N, K)
    m.scales[:] = e8m0
    for k in (0, 1, 33, 256, 511):
        x = synth.f32_to_bf16_bits(np.eye(1, K, k, dtype=np.float32)[0])
        assert np.array_equal(gemv_fp4(m, x, pkg.OUT_F32), oracle.mxfp4_gemv(m.codes, m.scales, x)), k
    # random x: at 2^125 keep |y| inside the fp32 / bf16 range
    x = synth.moe_token(64, K)
    if e8m0 == 252:
        x = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(x) * np.float32(2.0 ** -12))
    ref = oracle.mxfp4_gemv(m.codes, m.scales, x)
    assert_f32_close(gemv_fp4(m, x, pkg.OUT_F32), ref, what="f32 e8m0=%d" % e8m0)


def _pool(seed, E, H, F):
    ex = [synth.expert(seed, e, H, F) for e in range(E)]
    st = lambda f: np.stack([f(e) for e in ex])  # noqa: E731
    return (st(lambda e: e.gate.codes), st(lambda e: e.gate.scales), st(lambda e: e.up.codes),
            st(lambda e: e.up.scales), st(lambda e: e.down.codes), st(lambda e: e.down.scales))


def _pack_pool(pool, E, H, F):
    gc, gs, uc, us, dc, ds = pool
    pg = weights.pack_mxfp4(gc.reshape(E * F, H // 2), gs.reshape(E * F, H // 32), DEV)
    pu = weights.pack_mxfp4(uc.reshape(E * F, H // 2), us.reshape(E * F, H // 32), DEV)
    pd = weights.pack_mxfp4(dc.reshape(E * H, F // 2), ds.reshape(E * H, F // 32), DEV)
    return pg, pu, pd


def run_moe(packed, E, H, F, x, ids, w, out_dtype, workspace=None):
    pg, pu, pd = packed
    y = pkg.moe_expert_gemv_run(pg, pu, pd, E, H, F, weights.to_device(x, DEV),
                                weights.to_device(ids, DEV), weights.to_device(w, DEV),
                                workspace=workspace, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return to_np(y)


# two cases have more rowblocks of H than a GPU has CUs (the fused down
# projection's workgroups then take two rowblocks each in turn); the last
# case stages more h than fits in LDS, so it takes the two-launch down
# projection plus combine instead of the fused one
@pytest.mark.parametrize("E,H,F,top_k", [(6, 256, 512, 3), (4, 96, 160, 4), (9, 1024, 256, 1),
                                         (5, 5120, 256, 3), (9, 4160, 512, 7),
                                         (5, 64, 12288, 4)])
def test_moe_small(E, H, F, top_k):
    note("moe E=%d H=%d F=%d top_k=%d" % (E, H, F, top_k))
    pool = _pool(70, E, H, F)
    x = synth.moe_token(71, H)
    ids, w = synth.router(72, E, top_k)
    ref = oracle.moe(*pool, x, ids, w)
    packed = _pack_pool(pool, E, H, F)
    assert_f32_close(run_moe(packed, E, H, F, x, ids, w, pkg.OUT_F32), ref, what="f32")
    assert_bf16_close(run_moe(packed, E, H, F, x, ids, w, pkg.OUT_BF16), ref, what="bf16")


def test_moe_invalid_id_and_empty():
    E, H, F = 5, 128, 96
    pool = _pool(73, E, H, F)
    packed = _pack_pool(pool, E, H, F)
    x = synth.moe_token(74, H)
    ids = np.array([2, 7, 0], dtype=np.int32)  # 7 is out of range: contributes nothing
    w = np.array([0.5, 0.3, 0.2], dtype=np.float32)
    ws = torch.empty(pkg.moe_workspace_bytes(3, H, F), dtype=torch.uint8, device=DEV)
    got = run_moe(packed, E, H, F, x, ids, w, pkg.OUT_F32, workspace=ws)
    status_off = 4 * 3 * (H + F)
    assert int(ws[status_off:status_off + 4].view(torch.int32).item()) == 1
    ref = oracle.moe(*pool, x, ids, w)
    assert_f32_close(got, ref, what="invalid id")
    # a valid call rewrites the status word to 0
    run_moe(packed, E, H, F, x, ids[[0, 2]], w[[0, 2]], pkg.OUT_F32,
            workspace=ws[:pkg.moe_workspace_bytes(2, H, F)])
    status_off2 = 4 * 2 * (H + F)
    assert int(ws[status_off2:status_off2 + 4].view(torch.int32).item()) == 0
    # top_k = 0: y = 0
    y0 = run_moe(packed, E, H, F, x, np.zeros(0, np.int32), np.zeros(0, np.float32), pkg.OUT_F32)
    assert not np.any(y0)


def test_moe_permutation_invariance():
    E, H, F = 8, 256, 256
    pool = _pool(75, E, H, F)
    packed = _pack_pool(pool, E, H, F)
    x = synth.moe_token(76, H)
    ids, w = synth.router(77, E, 4)
    p = np.array([3, 1, 0, 2])
    a = run_moe(packed, E, H, F, x, ids, w, pkg.OUT_F32)
    b = run_moe(packed, E, H, F, x, ids[p], w[p], pkg.OUT_F32)
    ref = oracle.moe(*pool, x, ids, w)
    assert_f32_close(a, ref)
    assert_f32_close(b, ref)


def test_moe_routed_expert_workload_full():
    """The MoE workload at full size: 384 experts, hidden 7168, expert FFN
    2048, top-16 by a seeded router.  The 16 selected experts hold the seeded
    synthetic weights; every other expert of the 384 is filled with random
    bytes (random codes and scale bytes, NaN scales included), so reading a
    wrong expert changes the result."""
    E, H, F, top_k = 384, 7168, 2048, 16
    note("moe full E=%d H=%d F=%d top_k=%d" % (E, H, F, top_k))
    ids, w = synth.router(80, E, top_k)
    x = synth.moe_token(81, H)
    g = torch.Generator(device=DEV)
    g.manual_seed(82)
    bg = pkg.packed_bytes(FP4, E * F, H)
    bd = pkg.packed_bytes(FP4, E * H, F)
    pg = torch.randint(0, 256, (bg,), dtype=torch.uint8, device=DEV, generator=g)
    pu = torch.randint(0, 256, (bg,), dtype=torch.uint8, device=DEV, generator=g)
    pd = torch.randint(0, 256, (bd,), dtype=torch.uint8, device=DEV, generator=g)
    eg, ed = bg // E, bd // E
    sel = []
    for e in ids.tolist():
        ex = synth.expert(83, e, H, F)
        pkg.qgemv_pack(FP4, F, H, weights.to_device(ex.gate.codes, DEV),
                       weights.to_device(ex.gate.scales, DEV), out=pg[e * eg:(e + 1) * eg])
        pkg.qgemv_pack(FP4, F, H, weights.to_device(ex.up.codes, DEV),
                       weights.to_device(ex.up.scales, DEV), out=pu[e * eg:(e + 1) * eg])
        pkg.qgemv_pack(FP4, H, F, weights.to_device(ex.down.codes, DEV),
                       weights.to_device(ex.down.scales, DEV), out=pd[e * ed:(e + 1) * ed])
        sel.append(ex)
    got = run_moe((pg, pu, pd), E, H, F, x, ids, w, pkg.OUT_BF16)
    note("  gpu done; oracle over the 16 selected experts")

    def one(s):
        ex = sel[s]
        pool = tuple(a[None] for a in (ex.gate.codes, ex.gate.scales, ex.up.codes, ex.up.scales,
                                       ex.down.codes, ex.down.scales))
        return oracle.moe(*pool, x, np.array([0], np.int32), w[s:s + 1])

    with ThreadPoolExecutor(max_workers=16) as pool:
        parts = list(pool.map(one, range(top_k)))
    ref = np.zeros(H)
    for p in parts:  # slot order, as the definition sums
        ref += p
    assert_bf16_close(got, ref, what="moe full")


# ------------------------------------------------------------ T positions at once
def run_moe_t(packed, E, H, F, X, ids, w, out_dtype, workspace=None):
    pg, pu, pd = packed
    Y = pkg.moe_expert_skinny_run(pg, pu, pd, E, H, F, weights.to_device(X, DEV),
                                  weights.to_device(ids, DEV), weights.to_device(w, DEV),
                                  workspace=workspace, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return to_np(Y)


def _routes(seed, E, top_k, T):
    ids, w = zip(*[synth.router(seed, E, top_k, item=t) for t in range(T)])
    return np.stack(ids), np.stack(w)


def _tokens(seed, H, T):
    return np.stack([synth.moe_token(seed, H, item=t) for t in range(T)])


# experts shared across positions; H not a multiple of the 256-k tile; 320
# rowblocks of H; F at its maximum and H at its maximum (one position per
# group); every expert chosen by all 32 positions (8 groups of 4 per expert);
# T = 1
@pytest.mark.parametrize("E,H,F,top_k,T", [(6, 256, 512, 3, 5), (4, 96, 160, 4, 3),
                                           (9, 1024, 256, 2, 16), (5, 5120, 256, 3, 2),
                                           (3, 64, 12288, 2, 4), (4, 24576, 64, 2, 3),
                                           (6, 512, 256, 6, 32), (40, 256, 128, 8, 1)])
def test_moe_positions(E, H, F, top_k, T):
    note("moe positions E=%d H=%d F=%d top_k=%d T=%d" % (E, H, F, top_k, T))
    pool = _pool(90, E, H, F)
    X = _tokens(91, H, T)
    ids, w = _routes(92, E, top_k, T)
    ref = oracle.moe_positions(*pool, X, ids, w)
    packed = _pack_pool(pool, E, H, F)
    assert_f32_close(run_moe_t(packed, E, H, F, X, ids, w, pkg.OUT_F32), ref, what="f32")
    assert_bf16_close(run_moe_t(packed, E, H, F, X, ids, w, pkg.OUT_BF16), ref, what="bf16")


def test_moe_positions_invalid_duplicate_and_empty():
    E, H, F, T = 5, 128, 96, 3
    note("moe positions invalid ids, duplicates, top_k = 0")
    pool = _pool(93, E, H, F)
    packed = _pack_pool(pool, E, H, F)
    X = _tokens(94, H, T)
    # 7 and -1 are out of range; a position may repeat an expert
    ids = np.array([[2, 7, 0], [1, 1, 4], [-1, 3, 3]], dtype=np.int32)
    w = np.array([[0.5, 0.3, 0.2], [0.6, 0.1, 0.3], [0.2, 0.2, 0.6]], dtype=np.float32)
    ws = torch.empty(pkg.moe_skinny_workspace_bytes(T, 3, H, F), dtype=torch.uint8, device=DEV)
    got = run_moe_t(packed, E, H, F, X, ids, w, pkg.OUT_F32, workspace=ws)
    status_off = 4 * T * 3 * (H + F)
    assert int(ws[status_off:status_off + 4].view(torch.int32).item()) == 1
    assert_f32_close(got, oracle.moe_positions(*pool, X, ids, w), what="invalid id")
    ok = np.array([[2, 0], [1, 4], [3, 3]], dtype=np.int32)
    wok = w[:, :2].copy()
    got = run_moe_t(packed, E, H, F, X, ok, wok, pkg.OUT_F32, workspace=ws)
    assert int(ws[4 * T * 2 * (H + F):4 * T * 2 * (H + F) + 4].view(torch.int32).item()) == 0
    assert_f32_close(got, oracle.moe_positions(*pool, X, ok, wok), what="valid")
    y0 = run_moe_t(packed, E, H, F, X, np.zeros((T, 0), np.int32), np.zeros((T, 0), np.float32),
                   pkg.OUT_F32)
    assert y0.shape == (T, H) and not np.any(y0)


def test_moe_positions_rows_are_single_tokens():
    """Row t of a pass equals the single-token layer on X[t], ids[t], w[t]
    (both checked against the oracle; the kernels differ, so not bitwise),
    and reordering the positions reorders the rows bit for bit (the groups
    depend on the positions only through their ids)."""
    E, H, F, top_k, T = 12, 512, 256, 4, 6
    pool = _pool(95, E, H, F)
    packed = _pack_pool(pool, E, H, F)
    X = _tokens(96, H, T)
    ids, w = _routes(97, E, top_k, T)
    Y = run_moe_t(packed, E, H, F, X, ids, w, pkg.OUT_F32)
    for t in range(T):
        ref = oracle.moe(*pool, X[t], ids[t], w[t])
        assert_f32_close(Y[t], ref, what="pass row %d" % t)
        assert_f32_close(run_moe(packed, E, H, F, X[t], ids[t], w[t], pkg.OUT_F32), ref,
                         what="single token %d" % t)
    perm = np.array([5, 2, 0, 4, 1, 3])
    Yp = run_moe_t(packed, E, H, F, X[perm], ids[perm], w[perm], pkg.OUT_F32)
    assert np.array_equal(Yp, Y[perm])


def test_moe_positions_full():
    """The verification tile through the MoE layer at full size: 384 experts,
    hidden 7168, expert FFN 2048, top-16 per position, 16 positions with
    independent seeded routes.  Every expert holds seeded codes and E8M0
    scales (118..128); positions 0, 7 and 15 are checked against the oracle
    and every row against the single-token layer on the GPU."""
    E, H, F, top_k, T = 384, 7168, 2048, 16, 16
    note("moe positions full E=%d H=%d F=%d top_k=%d T=%d" % (E, H, F, top_k, T))
    g = torch.Generator(device=DEV)
    g.manual_seed(98)

    def canon(rows, K):
        codes = torch.randint(0, 256, (E * rows, K // 2), dtype=torch.uint8, device=DEV,
                              generator=g)
        scales = torch.randint(118, 129, (E * rows, K // 32), dtype=torch.uint8, device=DEV,
                               generator=g)
        return codes, scales

    cg, cu, cd = canon(F, H), canon(F, H), canon(H, F)
    packed = tuple(pkg.qgemv_pack(FP4, E * rows, K, c, s)
                   for (c, s), rows, K in ((cg, F, H), (cu, F, H), (cd, H, F)))
    X = _tokens(99, H, T)
    ids, w = _routes(100, E, top_k, T)
    Y = run_moe_t(packed, E, H, F, X, ids, w, pkg.OUT_BF16)
    Yf = run_moe_t(packed, E, H, F, X, ids, w, pkg.OUT_F32)
    note("  %d distinct experts over %d pairs" % (len(np.unique(ids)), ids.size))
    for t in range(T):
        y1 = run_moe(packed, E, H, F, X[t], ids[t], w[t], pkg.OUT_F32)
        assert_f32_close(Yf[t], y1, what="row %d vs single token" % t)
    note("  rows match the single-token layer; oracle for positions 0, 7, 15")

    def one(args):
        t, s = args
        e = int(ids[t, s])
        pool = tuple(a[e * n:(e + 1) * n].cpu().numpy()[None] for (a, n) in (
            (cg[0], F), (cg[1], F), (cu[0], F), (cu[1], F), (cd[0], H), (cd[1], H)))
        return oracle.moe(*pool, X[t], np.array([0], np.int32), w[t, s:s + 1])

    for t in (0, 7, 15):
        with ThreadPoolExecutor(max_workers=16) as ex:
            parts = list(ex.map(one, [(t, s) for s in range(top_k)]))
        ref = np.zeros(H)
        for p in parts:  # slot order, as the definition sums
            ref += p
        assert_bf16_close(Y[t], ref, what="position %d" % t)
