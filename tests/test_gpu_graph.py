"""HIP-graph capture of the calls that launch several kernels or read their
routing from the device: the T-position MoE layer (its grouping kernel
writes the records the expert kernels read), the M = 16 grouped verification
pass, the int8 row-scale and affine GEMVs and the affine 16-row product.  Each captured graph is
replayed several times with eager work and synchronizations in between, and
every replay is compared bit for bit with the eager call on the same
inputs; for the MoE the router output is changed in place between replays,
as a decode loop would."""
import numpy as np
import pytest
import torch

import quantized_weight_decode_dequant_amd as pkg
from quantized_weight_decode_dequant_amd import synth, weights, workloads
from helpers import note

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _replay_matches(g, out, eager_fn, prepare=None, reps=4):
    for rep in range(reps):
        if prepare is not None:
            prepare(rep)
        torch.cuda.synchronize()
        ref = eager_fn().clone()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d differs from the eager call" % rep
        _ = torch.randn(1000, device=DEV).sum().item()  # unrelated eager work in between


def test_graph_moe_positions_changing_routes():
    E, H, F, top_k, T = 24, 1024, 512, 4, 8
    note("graph moe positions E=%d H=%d F=%d top_k=%d T=%d" % (E, H, F, top_k, T))
    g = torch.Generator(device=DEV)
    g.manual_seed(130)

    def stack(rows, K):
        c = torch.randint(0, 256, (E * rows, K // 2), dtype=torch.uint8, device=DEV, generator=g)
        s = torch.randint(118, 129, (E * rows, K // 32), dtype=torch.uint8, device=DEV, generator=g)
        return pkg.qgemv_pack(pkg.FMT_MXFP4_G32, E * rows, K, c, s)

    pg, pu, pd = stack(F, H), stack(F, H), stack(H, F)
    X = weights.to_device(np.stack([synth.moe_token(131, H, item=t) for t in range(T)]), DEV)
    routes = [[synth.router(132, E, top_k, item=r * T + t) for t in range(T)] for r in range(5)]
    ids = torch.empty(T, top_k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, top_k, dtype=torch.float32, device=DEV)

    def set_route(r):
        ids.copy_(torch.from_numpy(np.stack([a for a, _ in routes[r]])))
        w.copy_(torch.from_numpy(np.stack([b for _, b in routes[r]])))

    set_route(0)
    ws = torch.empty(pkg.moe_skinny_workspace_bytes(T, top_k, H, F), dtype=torch.uint8, device=DEV)
    Y = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    Ye = torch.empty_like(Y)
    ws_e = torch.empty_like(ws)
    run = lambda out, wsp: pkg.moe_expert_skinny_run(pg, pu, pd, E, H, F, X, ids, w,  # noqa: E731
                                                      workspace=wsp, Y=out)
    graph = workloads.capture_graph(lambda: run(Y, ws))
    _replay_matches(graph, Y, lambda: run(Ye, ws_e), prepare=lambda rep: set_route(rep + 1))


def test_graph_verification_pass_m16():
    note("graph M=16 grouped pass")
    shapes = [(256, 4096), (1024, 4096), (64, 12288), (17, 320)]
    entries = []
    for i, (N, K) in enumerate(shapes):
        m = synth.q4_matrix(133, N, K, item=i)
        p = weights.pack_q4(m, DEV)
        X = weights.to_device(synth.activations(134, 16, K, item=i), DEV)
        entries.append((p, N, K, X, torch.empty(16, N, dtype=torch.bfloat16, device=DEV)))
    plan = pkg.qg_batch_plan_build(pkg.FMT_Q4_ASYM_G64, 16, entries)
    pkg.qg_batch_run(plan)
    torch.cuda.synchronize()
    eager = [e[4].clone() for e in entries]
    graph = workloads.capture_graph(lambda: pkg.qg_batch_run(plan))
    for rep in range(4):
        for e in entries:
            e[4].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for e, ref in zip(entries, eager):
            assert torch.equal(e[4], ref), "replay %d differs" % rep
        _ = torch.randn(1000, device=DEV).sum().item()


@pytest.mark.parametrize("kind", ["q8row", "affine3", "affine8"])
def test_graph_weight_only_gemv(kind):
    N, K = 3000, 4096
    note("graph gemv %s" % kind)
    if kind == "q8row":
        m = synth.q8row_matrix(135, N, K)
        fmt, packed = pkg.FMT_Q8_ROW, weights.pack_q8row(m, DEV)
    else:
        bits = int(kind[-1])
        m = synth.affine_matrix(135, N, K, bits, 64, bits == 3)
        fmt, packed = pkg.affine_format(bits, 64, bits == 3), weights.pack_affine(m, DEV)
    x = weights.to_device(synth.activations(136, 1, K)[0], DEV)
    y = torch.empty(N, dtype=torch.float32, device=DEV)
    ye = torch.empty_like(y)
    run = lambda out: pkg.qgemv_run(fmt, packed, N, K, x, y=out, out_dtype=pkg.OUT_F32)  # noqa: E731
    graph = workloads.capture_graph(lambda: run(y))

    def perturb(rep):
        x.copy_(weights.to_device(synth.activations(137, 1, K, item=rep)[0], DEV))

    _replay_matches(graph, y, lambda: run(ye), prepare=perturb)


@pytest.mark.parametrize("bits", [2, 5])
def test_graph_affine_skinny(bits):
    """The affine verification product (16 rows) captured in a HIP graph: each
    replay, with a new X staged between replays, equals the eager call on the
    same X."""
    M, N, K = 16, 2000, 4096
    note("graph affine skinny bits=%d" % bits)
    m = synth.affine_matrix(138, N, K, bits, 64, False)
    fmt, packed = pkg.affine_format(bits, 64, False), weights.pack_affine(m, DEV)
    X = weights.to_device(synth.activations(139, M, K), DEV)
    Y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    Ye = torch.empty_like(Y)
    run = lambda out: pkg.qgemm_skinny_run(fmt, packed, M, N, K, X, Y=out, out_dtype=pkg.OUT_F32)  # noqa: E731
    graph = workloads.capture_graph(lambda: run(Y))

    def perturb(rep):
        X.copy_(weights.to_device(synth.activations(140, M, K, item=rep), DEV))

    _replay_matches(graph, Y, lambda: run(Ye), prepare=perturb)
