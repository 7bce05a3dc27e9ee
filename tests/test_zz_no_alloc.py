"""GPU test of moe_expert_gemv_run_noalloc, the MoE call that allocates
nothing (its workspace is the library's own device array).

Two calls in a row through the C ABI, the second with a smaller layer (and an
out-of-range expert id), each checked bit for bit against
moe_expert_gemv_run with a caller workspace (the same kernels), for bf16
and fp32 output, with the invalid-id status word; the first also against
the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import quantized_weight_decode_dequant_amd as pkg
from quantized_weight_decode_dequant_amd import synth, weights
from helpers import assert_f32_close, note, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
FP4 = pkg.FMT_MXFP4_G32


def _layer(seed, E, H, F):
    ex = [synth.expert(seed, e, H, F) for e in range(E)]
    st = lambda f: np.stack([f(e) for e in ex])  # noqa: E731
    pool = (st(lambda e: e.gate.codes), st(lambda e: e.gate.scales), st(lambda e: e.up.codes),
            st(lambda e: e.up.scales), st(lambda e: e.down.codes), st(lambda e: e.down.scales))
    gc, gs, uc, us, dc, ds = pool
    packed = (weights.pack_mxfp4(gc.reshape(E * F, H // 2), gs.reshape(E * F, H // 32), DEV),
              weights.pack_mxfp4(uc.reshape(E * F, H // 2), us.reshape(E * F, H // 32), DEV),
              weights.pack_mxfp4(dc.reshape(E * H, F // 2), ds.reshape(E * H, F // 32), DEV))
    return pool, packed


def _both(packed, E, H, F, x, ids, w, out_dtype):
    """(noalloc y, noalloc status, workspace-call y, workspace status)."""
    pg, pu, pd = packed
    xd, idd, wd = (weights.to_device(a, DEV) for a in (x, ids, w))
    st = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    y0 = pkg.moe_expert_gemv_run_noalloc(pg, pu, pd, E, H, F, xd, idd, wd, status=st,
                                         out_dtype=out_dtype)
    ws = torch.empty(pkg.moe_workspace_bytes(len(ids), H, F), dtype=torch.uint8, device=DEV)
    y1 = pkg.moe_expert_gemv_run(pg, pu, pd, E, H, F, xd, idd, wd, workspace=ws,
                                 out_dtype=out_dtype)
    torch.cuda.synchronize()
    off = 4 * len(ids) * (H + F)
    return y0, int(st.item()), y1, int(ws[off:off + 4].view(torch.int32).item())


def test_noalloc_moe_matches_workspace_call_twice():
    # call 1: the hidden and expert sizes of the routed-expert workload, top-16
    E, H, F = 20, 7168, 2048
    note("noalloc moe call 1: E=%d H=%d F=%d top_k=16" % (E, H, F))
    pool, packed = _layer(90, E, H, F)
    x = synth.moe_token(91, H)
    ids, w = synth.router(92, E, 16)
    for out in (pkg.OUT_BF16, pkg.OUT_F32):
        y0, s0, y1, s1 = _both(packed, E, H, F, x, ids, w, out)
        assert torch.equal(y0, y1), "call 1 differs from moe_expert_gemv_run (out %d)" % out
        assert s0 == 0 and s1 == 0
    assert_f32_close(to_np(y0), oracle.moe(*pool, x, ids, w), what="call 1 vs oracle")
    # call 2: a smaller layer, with an expert id out of range; the array still
    # holds call 1's (larger) contents
    E2, H2, F2 = 6, 1024, 512
    note("noalloc moe call 2: E=%d H=%d F=%d top_k=3" % (E2, H2, F2))
    pool2, packed2 = _layer(93, E2, H2, F2)
    x2 = synth.moe_token(94, H2)
    ids2 = np.array([4, 9, 1], dtype=np.int32)  # 9 is out of range: contributes nothing
    w2 = np.array([0.5, 0.3, 0.2], dtype=np.float32)
    for out in (pkg.OUT_F32, pkg.OUT_BF16):
        y0, s0, y1, s1 = _both(packed2, E2, H2, F2, x2, ids2, w2, out)
        assert torch.equal(y0, y1), "call 2 differs from moe_expert_gemv_run (out %d)" % out
        assert s0 == 1 and s1 == 1
    assert_f32_close(to_np(_both(packed2, E2, H2, F2, x2, ids2, w2, pkg.OUT_F32)[0]),
                     oracle.moe(*pool2, x2, ids2, w2), what="call 2 vs oracle")


def test_noalloc_moe_rejects_oversized_layer():
    """A layer whose workspace exceeds the array is refused before any launch."""
    E, H, F, k = 16, 24576, 12288, 16
    assert pkg.moe_workspace_bytes(k, H, F) > pkg.MOE_NOALLOC_SCRATCH_BYTES
    g = torch.empty(pkg.packed_bytes(FP4, E * F, H), dtype=torch.uint8, device=DEV)
    d = torch.empty(pkg.packed_bytes(FP4, E * H, F), dtype=torch.uint8, device=DEV)
    x = torch.zeros(H, dtype=torch.bfloat16, device=DEV)
    ids = torch.arange(k, dtype=torch.int32, device=DEV)
    w = torch.ones(k, dtype=torch.float32, device=DEV)
    with pytest.raises(pkg.QGError) as e:
        pkg.moe_expert_gemv_run_noalloc(g, g, d, E, H, F, x, ids, w)
    assert e.value.status == pkg.QG_ESIZE
