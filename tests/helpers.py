"""Comparison helpers for the GPU parity tests.

Tolerances (the dequant paths accumulate in fp32; the oracle is fp64):
 * fp32 output: max_i |got_i - ref_i| / max(|ref_i|, 1e-2 * rms(ref)) <= 2e-3.
   The floor keeps outputs that cancel to nearly zero from dominating a
   relative measure; it is 1% of the typical output magnitude.
 * bf16 output: every element within one bf16 ulp of the exact value (or the
   same floor, scaled by 2e-3), and, for vectors of at least 64 elements, the
   distance to the correctly rounded exact value (bf16 round-to-nearest-even
   of the reference) at most 2e-3 in relative L2.  A literal 2e-3 bound
   against the exact value is below bf16's own rounding: elementwise it
   reaches 2^-8 relative, and even the L2 of the rounding alone is about
   1.6e-3 (up to 2.1e-3 on 100 outputs), so the correctly rounded answer
   itself would fail it.
 * integer outputs: bit-exact.
"""
import sys

import numpy as np

TOL = 2e-3
FLOOR_FRAC = 1e-2


def note(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def rms(a):
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    floor = FLOOR_FRAC * rms(ref)
    den = np.maximum(np.abs(ref), floor if floor > 0 else 1e-30)
    return float(np.max(np.abs(got - ref) / den)) if ref.size else 0.0


def assert_f32_close(got, ref, tol=TOL, what=""):
    assert np.all(np.isfinite(got)), what
    e = rel_err(got, ref)
    assert e <= tol, "%s: max rel err %.3g > %.3g" % (what, e, tol)
    return e


def bf16_ulp(ref):
    a = np.maximum(np.abs(np.asarray(ref, dtype=np.float64)), 1e-38)
    return np.exp2(np.floor(np.log2(a)) - 7)


def bf16_round(a):
    """float64 -> nearest bf16 value (round-to-nearest-even, via float32),
    as float64."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def assert_bf16_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), what
    lim = np.maximum(bf16_ulp(ref), TOL * FLOOR_FRAC * rms(ref))
    bad = np.abs(got - ref) > lim
    assert not bad.any(), "%s: %d elements beyond 1 bf16 ulp, first at %s (got %r ref %r)" % (
        what, int(bad.sum()), np.argwhere(bad)[0], got[bad][0], ref[bad][0])
    rounded = bf16_round(ref)
    l2 = float(np.linalg.norm(got - rounded) / max(np.linalg.norm(ref), 1e-300))
    if ref.size >= 64:
        assert l2 <= TOL, "%s: rel L2 %.3g" % (what, l2)
    return l2


def assert_same(got, want, what=""):
    """Bitwise equality of two device tensors; on a mismatch the message
    names how many elements differ, where, and their values."""
    import torch
    if torch.equal(got, want):
        return
    a, b = got.flatten(), want.flatten()
    if a.shape != b.shape:
        raise AssertionError("%s: shapes %s and %s" % (what, tuple(got.shape), tuple(want.shape)))
    if a.dtype in (torch.bfloat16, torch.float16):
        diff = a.view(torch.int16) != b.view(torch.int16)
    else:
        diff = a != b
    idx = torch.nonzero(diff).flatten()[:8].tolist()
    raise AssertionError("%s: %d of %d elements differ, first at %s: got %s want %s" % (
        what, int(diff.sum()), a.numel(), idx, a[idx].float().tolist(), b[idx].float().tolist()))


def to_np(t):
    """Device tensor -> float64 numpy (bf16/fp32 widen exactly)."""
    import torch
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.detach().cpu().numpy().astype(np.float64)
