"""Device-resident synthetic workloads (plumbing for the benchmark and tests).

The synthetic dense decode step: 36 layers of seven 4-bit group-64
projections (q 4096->4096, k and v 4096->1024, o 4096->4096, gate and up
4096->12288, down 12288->4096) plus an lm_head 4096->151936, about 4.26 GB of
packed weights, each projection with its own seeded activation vector; no
chaining between projections, no attention or norms -- only the GEMVs, whose
bytes set the decode ceiling (Uzu page, fange-kb.cn, section "Why batch-one
decoding is memory-bound").
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import _lib, roofline, synth, weights


@dataclass
class Gemv:
    item: int
    name: str
    N: int
    K: int
    packed: object          # uint8 device tensor
    x: object               # bf16 device tensor [K]
    y: object               # bf16 device tensor [N]
    X: object = None        # bf16 device tensor [M, K] for the skinny pass
    Y: object = None


@dataclass
class DecodeStep:
    gemvs: list = field(default_factory=list)
    seed: int = 0
    M: int = 0

    @property
    def weight_bytes(self) -> int:
        return int(sum(g.packed.numel() for g in self.gemvs))

    def algorithmic_bytes(self, M: int = 1) -> float:
        return float(sum(roofline.q4_gemm_bytes(M, g.N, g.K) for g in self.gemvs))

    def flops(self, M: int = 1) -> float:
        return float(sum(roofline.gemm_flops(M, g.N, g.K) for g in self.gemvs))


def build_decode_step(seed: int = 0, layers: int = synth.DECODE_LAYERS, device="cuda",
                      skinny_m: int = 0, log=None) -> DecodeStep:
    """Generate, upload and pack every projection of the decode step."""
    import torch
    step = DecodeStep(seed=seed, M=skinny_m)
    for item, name, N, K in synth.decode_step_shapes(layers):
        m = synth.q4_matrix(seed, N, K, item=item)
        packed = weights.pack_q4(m, device)
        del m
        x = weights.to_device(synth.activations(seed, 1, K, item=item)[0], device).view(torch.bfloat16)
        y = torch.empty(N, dtype=torch.bfloat16, device=device)
        g = Gemv(item, name, N, K, packed, x, y)
        if skinny_m:
            g.X = weights.to_device(synth.activations(seed + 1, skinny_m, K, item=item),
                                    device).view(torch.bfloat16)
            g.Y = torch.empty((skinny_m, N), dtype=torch.bfloat16, device=device)
        step.gemvs.append(g)
        if log and (item % 50 == 0 or name == "lm_head"):
            log("  packed %s (%d x %d)" % (name, N, K))
    torch.cuda.synchronize()
    return step


def verification_tile(seed: int, g: Gemv, M: int, device="cuda"):
    """The M-row bf16 activation tile of one projection for a verification
    pass (seeded per projection, independent of the M = 1 vector)."""
    import torch
    return weights.to_device(synth.activations(seed + 1, M, g.K, item=g.item), device).view(torch.bfloat16)


def run_step_eager(step: DecodeStep, stream=None):
    """One decode step: every GEMV of the step enqueued on the stream."""
    for g in step.gemvs:
        _lib.qgemv_run(_lib.FMT_Q4_ASYM_G64, g.packed, g.N, g.K, g.x, g.y, stream=stream)


def run_skinny_eager(step: DecodeStep, stream=None):
    """One verification pass: every projection against its M-row tile."""
    for g in step.gemvs:
        _lib.qgemm_skinny_run(_lib.FMT_Q4_ASYM_G64, g.packed, step.M, g.N, g.K, g.X, Y=g.Y,
                              stream=stream)


def capture_graph(fn):
    """Capture fn() (which enqueues on torch's current stream) into a HIP graph."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm the launch path outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_ms(fn, iters: int, warmup: int = 2) -> float:
    """Mean milliseconds per call of fn() on the current stream (HIP events
    around the whole loop, so back-to-back launch gaps are included)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def settle(fn, seconds: float, chunk: int = 20) -> int:
    """Run fn() untimed, `chunk` calls between synchronizations, until at least
    `seconds` of wall time have passed (a GPU coming out of a lighter load
    runs below its sustained clock for a fraction of a second); returns the
    number of calls."""
    import time
    import torch
    t0, n = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(chunk):
            fn()
        n += chunk
        torch.cuda.synchronize()
    return n


def time_graph_ms(fn, calls: int, reps: int = 5, settle_s: float = 0.2) -> float:
    """Mean milliseconds per call of fn() measured on the GPU: `calls`
    invocations captured into one HIP graph, the graph replayed `reps` times
    between HIP events (after `settle_s` seconds of untimed replays).  For
    kernels shorter than the host's launch path this times the device, not
    the Python binding."""
    import torch
    graph = capture_graph(lambda: [fn() for _ in range(calls)])
    graph.replay()
    torch.cuda.synchronize()
    settle(graph.replay, settle_s, chunk=4)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * calls)
    del graph
    return ms


class Int8Verify:
    """The 8-bit verification workload: a 16-row activation tile rotated and
    quantized to int8, then multiplied with 8-bit symmetric group-32 weights.
    The packed matrix is replicated `copies` times at distinct addresses so
    consecutive calls stream from HBM, not from the 256 MB last-level cache."""

    def __init__(self, seed: int, N: int, K: int, M: int = 16, copies: int = 40, device="cuda"):
        import torch
        self.N, self.K, self.M = N, K, M
        w = synth.q8_matrix(seed, N, K)
        base = weights.pack_q8(w, device)
        self.packed = [base] + [base.clone() for _ in range(copies - 1)]
        self.X = weights.to_device(synth.q8_activations(seed, M, K), device)
        self.signs = weights.to_device(synth.rotation_signs(seed, K), device)
        self.Xq = torch.empty((M, K), dtype=torch.int8, device=device)
        self.sx = torch.empty(M, dtype=torch.float32, device=device)
        self.Y = torch.empty((M, N), dtype=torch.bfloat16, device=device)
        self.i = 0

    def quantize(self):
        _lib.hadamard32_quant_run(self.X, self.signs, self.M, self.K, self.Xq, self.sx)

    def gemm(self):
        p = self.packed[self.i % len(self.packed)]
        self.i += 1
        _lib.qgemm_skinny_run(_lib.FMT_Q8_SYM_G32, p, self.M, self.N, self.K, self.Xq, self.sx,
                              Y=self.Y)


class MoeLayer:
    """One routed-expert MoE layer in MXFP4 (E experts, hidden H, expert FFN
    F): the whole pool packed on the device, codes uniform over the 16 E2M1
    codes and E8M0 scales uniform in 118..128, drawn with a seeded device
    generator; `routes` seeded router draws (top_k of E, softmax weights), a
    different one per call so the selected experts change between calls."""

    def __init__(self, seed: int, E: int, H: int, F: int, top_k: int, routes: int = 64,
                 device="cuda", T: int = 0):
        import numpy as np
        import torch
        self.E, self.H, self.F, self.top_k, self.T = E, H, F, top_k, T
        g = torch.Generator(device=device)
        g.manual_seed(seed)

        def stack(rows, K):
            codes = torch.randint(0, 256, (E * rows, K // 2), dtype=torch.uint8, device=device,
                                  generator=g)
            scales = torch.randint(118, 129, (E * rows, K // 32), dtype=torch.uint8,
                                   device=device, generator=g)
            out = _lib.qgemv_pack(_lib.FMT_MXFP4_G32, E * rows, K, codes, scales)
            del codes, scales
            return out

        self.gate = stack(F, H)
        self.up = stack(F, H)
        self.down = stack(H, F)
        if T == 0:
            # one token per call
            ids, ws = zip(*[synth.router(seed, E, top_k, item=r) for r in range(routes)])
            self.x = weights.to_device(synth.moe_token(seed, H), device)
            self.workspace = torch.empty(_lib.moe_workspace_bytes(top_k, H, F),
                                         dtype=torch.uint8, device=device)
            self.y = torch.empty(H, dtype=torch.bfloat16, device=device)
        else:
            # T positions per call, each with its own route
            ids, ws = zip(*[tuple(np.stack(a) for a in zip(*[
                synth.router(seed, E, top_k, item=r * T + t) for t in range(T)]))
                for r in range(routes)])
            self.x = weights.to_device(np.stack([synth.moe_token(seed, H, item=t)
                                                 for t in range(T)]), device)
            self.workspace = torch.empty(_lib.moe_skinny_workspace_bytes(T, top_k, H, F),
                                         dtype=torch.uint8, device=device)
            self.y = torch.empty(T, H, dtype=torch.bfloat16, device=device)
        self.ids_host = np.stack(ids)
        self.ids = weights.to_device(self.ids_host, device)
        self.w = weights.to_device(np.stack(ws), device)
        self.i = 0

    def distinct_experts(self) -> float:
        """Mean number of distinct experts per call over the route sets."""
        return float(np.mean([len(np.unique(r)) for r in self.ids_host]))

    def run(self):
        r = self.i % self.ids.shape[0]
        self.i += 1
        if self.T == 0:
            _lib.moe_expert_gemv_run(self.gate, self.up, self.down, self.E, self.H, self.F,
                                     self.x, self.ids[r], self.w[r], workspace=self.workspace,
                                     y=self.y)
        else:
            _lib.moe_expert_skinny_run(self.gate, self.up, self.down, self.E, self.H, self.F,
                                       self.x, self.ids[r], self.w[r], workspace=self.workspace,
                                       Y=self.y)
