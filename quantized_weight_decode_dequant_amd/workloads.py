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
