"""Upload canonical host weights (from ``synth``) to the device and pack them.

Plumbing only: host arrays become device tensors with torch, then the
library's qgemv_pack converts them into the packed layout; the canonical
device copies are released afterwards.
"""
from __future__ import annotations

import numpy as np

from . import _lib


def to_device(a: np.ndarray, device="cuda"):
    """numpy array -> device tensor with the same bytes (unsigned types are
    carried in the signed torch type of the same width)."""
    import torch
    view = {np.uint16: np.int16, np.uint32: np.int32, np.uint64: np.int64}.get(a.dtype.type)
    a = np.ascontiguousarray(a)
    if view is not None:
        a = a.view(view)
    return torch.from_numpy(a).to(device)


def pack_q4(m, device="cuda", stream=None):
    codes, scales, biases = to_device(m.codes, device), to_device(m.scales, device), to_device(m.biases, device)
    return _lib.qgemv_pack(_lib.FMT_Q4_ASYM_G64, m.codes.shape[0], m.codes.shape[1] * 8, codes,
                           scales, biases, stream=stream)


def pack_q8(m, device="cuda", stream=None):
    codes, scales = to_device(m.qw, device), to_device(m.sw, device)
    return _lib.qgemv_pack(_lib.FMT_Q8_SYM_G32, m.qw.shape[0], m.qw.shape[1], codes, scales,
                           stream=stream)


def pack_mxfp4(codes: np.ndarray, scales: np.ndarray, device="cuda", stream=None):
    """codes uint8 [rows, K/2], scales uint8 [rows, K/32]; stacked experts are
    passed as rows = E * N."""
    rows, K = codes.shape[0], codes.shape[1] * 2
    return _lib.qgemv_pack(_lib.FMT_MXFP4_G32, rows, K, to_device(codes, device),
                           to_device(scales, device), stream=stream)


def pack_q8row(m, device="cuda", stream=None):
    """Weight-only int8: codes int8 [N, K], scales float32 [N]."""
    return _lib.qgemv_pack(_lib.FMT_Q8_ROW, m.codes.shape[0], m.codes.shape[1],
                           to_device(m.codes, device), to_device(m.scales, device), stream=stream)


def pack_affine(m, device="cuda", stream=None):
    """Affine family (synth.AffineMatrix): codes uint8 [N, K], scales and
    biases uint16 [N, K/group]."""
    fmt = _lib.affine_format(m.bits, m.group, m.bf16_scales)
    return _lib.qgemv_pack(fmt, m.codes.shape[0], m.codes.shape[1], to_device(m.codes, device),
                           to_device(m.scales, device), to_device(m.biases, device),
                           stream=stream)
