"""Thin Python binding of the C ABI in include/qgemv.h.

Argument marshalling only: tensors are passed to the library as raw device
pointers with the current HIP stream, every step of the computation runs in
the library's kernels.  PyTorch supplies device memory and streams; output
tensors the caller does not provide are allocated here with torch.

The binding refuses to run without the compiled library: there is no
fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

from .build import LIB_PATH

FMT_Q4_ASYM_G64 = 1
FMT_Q8_SYM_G32 = 2
FMT_MXFP4_G32 = 3
FMT_Q8_ROW = 4


def affine_format(bits: int, group: int, bf16_scales: bool = False) -> int:
    """QG_FMT_AFFINE(bits, group, bf16_scales) of qgemv.h."""
    gc = {32: 0, 64: 1, 128: 2}.get(group, 3)
    return 0x100 | ((bits & 0xF) << 4) | (gc << 2) | (1 if bf16_scales else 0)

OUT_BF16 = 0
OUT_F32 = 1
OUT_I32_GROUPS = 2

KERNEL_AUTO = 0
KERNEL_VALU = 1
KERNEL_MFMA = 2

QG_OK = 0
QG_EINVAL = -1
QG_ESHAPE = -2
QG_EALIGN = -3
QG_ESIZE = -4
QG_EUNSUPPORTED = -5
QG_EHIP = -6
QG_EINTERNAL = -7

# every function include/qgemv.h declares
EXPORTS = (
    "qg_status_string",
    "qg_version",
    "qgemv_pack",
    "qgemv_run",
    "qgemm_skinny_run",
    "hadamard32_quant_run",
    "qg_moe_workspace_bytes",
    "moe_expert_gemv_run",
    "moe_expert_gemv_run_noalloc",
    "qg_moe_skinny_workspace_bytes",
    "moe_expert_skinny_run",
    "qg_batch_worklist_bytes",
    "qg_batch_plan_build",
    "qg_batch_run",
    "qg_plain_read",
)


class GemvDesc(C.Structure):
    """struct qg_gemv_desc"""
    _fields_ = [("packed", C.c_void_p), ("packed_bytes", C.c_size_t), ("N", C.c_int64),
                ("K", C.c_int64), ("x", C.c_void_p), ("y", C.c_void_p)]


class BatchPlan(C.Structure):
    """struct qg_batch_plan"""
    _fields_ = [("fmt", C.c_int32), ("M", C.c_int32), ("count", C.c_int32),
                ("out_dtype", C.c_int32), ("grid", C.c_int32), ("kmax", C.c_int32),
                ("kernel", C.c_int32), ("reserved1", C.c_int32), ("worklist", C.c_void_p),
                ("worklist_bytes", C.c_size_t)]

_lock = threading.Lock()
_lib = None


class QGError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s" % (where, status_string(status)))


def raw():
    """The loaded library with argument types set (loads on first use)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    "libqgemv.so is not built (%s); run __graft_entry__.build() or "
                    "python -m quantized_weight_decode_dequant_amd.build" % LIB_PATH)
            lib = C.CDLL(LIB_PATH)
            i64, p, i, sz = C.c_int64, C.c_void_p, C.c_int, C.c_size_t
            lib.qg_status_string.argtypes = [i]
            lib.qg_status_string.restype = C.c_char_p
            lib.qg_version.argtypes = []
            lib.qg_version.restype = i
            lib.qgemv_pack.argtypes = [i, i64, i64, p, p, p, p, C.POINTER(sz), p]
            lib.qgemv_pack.restype = i
            lib.qgemv_run.argtypes = [i, p, sz, i64, i64, p, p, i, p]
            lib.qgemv_run.restype = i
            lib.qgemm_skinny_run.argtypes = [i, p, sz, i64, i64, i64, p, p, p, i, p]
            lib.qgemm_skinny_run.restype = i
            lib.hadamard32_quant_run.argtypes = [p, p, i64, i64, p, p, p]
            lib.hadamard32_quant_run.restype = i
            lib.qg_moe_workspace_bytes.argtypes = [i64, i64, i64]
            lib.qg_moe_workspace_bytes.restype = sz
            lib.moe_expert_gemv_run.argtypes = [p, p, p, sz, sz, sz, i64, i64, i64, p, i, p, p,
                                                p, sz, p, i, p]
            lib.moe_expert_gemv_run.restype = i
            lib.moe_expert_gemv_run_noalloc.argtypes = [p, p, p, sz, sz, sz, i64, i64, i64, p, i,
                                                        p, p, p, p, i, p]
            lib.moe_expert_gemv_run_noalloc.restype = i
            lib.qg_moe_skinny_workspace_bytes.argtypes = [i64, i64, i64, i64]
            lib.qg_moe_skinny_workspace_bytes.restype = sz
            lib.moe_expert_skinny_run.argtypes = [p, p, p, sz, sz, sz, i64, i64, i64, i64, p, i,
                                                  p, p, p, sz, p, i, p]
            lib.moe_expert_skinny_run.restype = i
            lib.qg_batch_worklist_bytes.argtypes = [C.c_int32]
            lib.qg_batch_worklist_bytes.restype = sz
            lib.qg_batch_plan_build.argtypes = [i, i64, C.c_int32, C.POINTER(GemvDesc), i, i, p, sz,
                                                C.POINTER(BatchPlan), p]
            lib.qg_batch_plan_build.restype = i
            lib.qg_batch_run.argtypes = [C.POINTER(BatchPlan), p]
            lib.qg_batch_run.restype = i
            lib.qg_plain_read.argtypes = [p, sz, p, i, p]
            lib.qg_plain_read.restype = i
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    return raw().qg_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != QG_OK:
        raise QGError(status, where)


# ------------------------------------------------------------------ torch glue
def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return C.c_void_p(t.data_ptr())


def _out_torch_dtype(out_dtype):
    torch = _torch()
    return {OUT_BF16: torch.bfloat16, OUT_F32: torch.float32, OUT_I32_GROUPS: torch.int32}[out_dtype]


# ------------------------------------------------------------------ API
def packed_bytes(fmt: int, rows: int, K: int) -> int:
    n = C.c_size_t(0)
    _check(raw().qgemv_pack(fmt, rows, K, None, None, None, None, C.byref(n), None), "qgemv_pack")
    return n.value


def qgemv_pack(fmt: int, rows: int, K: int, codes, scales, biases=None, out=None, stream=None):
    """Pack canonical device tensors; returns the packed uint8 device tensor."""
    torch = _torch()
    nbytes = packed_bytes(fmt, rows, K)
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=codes.device)
    cap = C.c_size_t(out.numel() * out.element_size())
    _check(raw().qgemv_pack(fmt, rows, K, _ptr(codes), _ptr(scales), _ptr(biases), _ptr(out),
                            C.byref(cap), _stream(stream)), "qgemv_pack")
    return out[:nbytes] if out.numel() != nbytes else out


def qgemv_run(fmt: int, packed, N: int, K: int, x, y=None, out_dtype: int = OUT_BF16,
              stream=None):
    torch = _torch()
    if y is None:
        y = torch.empty(N, dtype=_out_torch_dtype(out_dtype), device=x.device)
    _check(raw().qgemv_run(fmt, _ptr(packed), packed.numel(), N, K, _ptr(x), _ptr(y), out_dtype,
                           _stream(stream)), "qgemv_run")
    return y


def qgemm_skinny_run(fmt: int, packed, M: int, N: int, K: int, X, x_scales=None, Y=None,
                     out_dtype: int = OUT_BF16, stream=None):
    torch = _torch()
    if Y is None:
        shape = (M, N, K // 32) if out_dtype == OUT_I32_GROUPS else (M, N)
        Y = torch.empty(shape, dtype=_out_torch_dtype(out_dtype), device=X.device)
    _check(raw().qgemm_skinny_run(fmt, _ptr(packed), packed.numel(), M, N, K, _ptr(X),
                                  _ptr(x_scales), _ptr(Y), out_dtype, _stream(stream)),
           "qgemm_skinny_run")
    return Y


def hadamard32_quant_run(X, signs, M: int, K: int, Xq=None, x_scales=None, stream=None):
    torch = _torch()
    if Xq is None:
        Xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if x_scales is None:
        x_scales = torch.empty(M, dtype=torch.float32, device=X.device)
    _check(raw().hadamard32_quant_run(_ptr(X), _ptr(signs), M, K, _ptr(Xq), _ptr(x_scales),
                                      _stream(stream)), "hadamard32_quant_run")
    return Xq, x_scales


def moe_workspace_bytes(top_k: int, H: int, F: int) -> int:
    return raw().qg_moe_workspace_bytes(top_k, H, F)


def moe_expert_gemv_run(packed_gate, packed_up, packed_down, E: int, H: int, F: int, x,
                        expert_ids, expert_w, workspace=None, y=None, out_dtype: int = OUT_BF16,
                        stream=None):
    torch = _torch()
    top_k = int(expert_ids.numel())
    if workspace is None:
        workspace = torch.empty(moe_workspace_bytes(top_k, H, F), dtype=torch.uint8,
                                device=x.device)
    if y is None:
        y = torch.empty(H, dtype=_out_torch_dtype(out_dtype), device=x.device)
    _check(raw().moe_expert_gemv_run(_ptr(packed_gate), _ptr(packed_up), _ptr(packed_down),
                                     packed_gate.numel(), packed_up.numel(), packed_down.numel(),
                                     E, H, F, _ptr(x), top_k, _ptr(expert_ids), _ptr(expert_w),
                                     _ptr(workspace), workspace.numel(), _ptr(y), out_dtype,
                                     _stream(stream)), "moe_expert_gemv_run")
    return y


# the largest workspace moe_expert_gemv_run_noalloc serves (QG_MOE_NOALLOC_SCRATCH_BYTES)
MOE_NOALLOC_SCRATCH_BYTES = 2 << 20


def moe_expert_gemv_run_noalloc(packed_gate, packed_up, packed_down, E: int, H: int, F: int, x,
                                expert_ids, expert_w, status=None, y=None,
                                out_dtype: int = OUT_BF16, stream=None):
    """moe_expert_gemv_run on the library's own device array instead of a
    workspace; status: optional int32 device tensor [1] receiving the
    invalid-id flag."""
    torch = _torch()
    top_k = int(expert_ids.numel())
    if y is None:
        y = torch.empty(H, dtype=_out_torch_dtype(out_dtype), device=x.device)
    _check(raw().moe_expert_gemv_run_noalloc(
        _ptr(packed_gate), _ptr(packed_up), _ptr(packed_down), packed_gate.numel(),
        packed_up.numel(), packed_down.numel(), E, H, F, _ptr(x), top_k, _ptr(expert_ids),
        _ptr(expert_w), _ptr(status), _ptr(y), out_dtype, _stream(stream)),
        "moe_expert_gemv_run_noalloc")
    return y


def moe_skinny_workspace_bytes(T: int, top_k: int, H: int, F: int) -> int:
    return raw().qg_moe_skinny_workspace_bytes(T, top_k, H, F)


def moe_expert_skinny_run(packed_gate, packed_up, packed_down, E: int, H: int, F: int, X,
                          expert_ids, expert_w, workspace=None, Y=None,
                          out_dtype: int = OUT_BF16, stream=None):
    """X [T, H] bf16; expert_ids int32 / expert_w fp32 [T, top_k]; Y [T, H]."""
    torch = _torch()
    T = int(X.shape[0])
    top_k = int(expert_ids.shape[1]) if expert_ids.dim() == 2 else 0
    if tuple(expert_ids.shape) != (T, top_k) or tuple(expert_w.shape) != (T, top_k):
        raise ValueError("expert_ids and expert_w must be [T, top_k]")
    if workspace is None:
        workspace = torch.empty(moe_skinny_workspace_bytes(T, top_k, H, F), dtype=torch.uint8,
                                device=X.device)
    if Y is None:
        Y = torch.empty(T, H, dtype=_out_torch_dtype(out_dtype), device=X.device)
    _check(raw().moe_expert_skinny_run(_ptr(packed_gate), _ptr(packed_up), _ptr(packed_down),
                                       packed_gate.numel(), packed_up.numel(),
                                       packed_down.numel(), E, H, F, T, _ptr(X), top_k,
                                       _ptr(expert_ids), _ptr(expert_w), _ptr(workspace),
                                       workspace.numel(), _ptr(Y), out_dtype, _stream(stream)),
           "moe_expert_skinny_run")
    return Y


# ------------------------------------------------------------------ grouped launches
class Plan:
    """A built qg_batch_plan plus the device work list and the tensors its
    descriptors point at (kept alive as long as the plan)."""

    def __init__(self, plan, worklist, keep):
        self.plan = plan
        self.worklist = worklist
        self._keep = keep

    @property
    def grid(self) -> int:
        return self.plan.grid


def qg_batch_worklist_bytes(count: int) -> int:
    return raw().qg_batch_worklist_bytes(count)


def qg_batch_plan_build(fmt: int, M: int, entries, out_dtype: int = OUT_BF16, worklist=None,
                        stream=None, kernel: int = KERNEL_AUTO) -> Plan:
    """entries: sequence of (packed, N, K, x, y) with device tensors; x is bf16
    [M, K] ([K] for M = 1), y is [M, N] of the output type.  kernel: one of
    KERNEL_AUTO, KERNEL_VALU, KERNEL_MFMA."""
    torch = _torch()
    entries = list(entries)
    descs = (GemvDesc * len(entries))()
    keep = []
    for d, (packed, N, K, x, y) in zip(descs, entries):
        d.packed = _ptr(packed)
        d.packed_bytes = packed.numel()
        d.N, d.K = N, K
        d.x = _ptr(x)
        d.y = _ptr(y)
        keep.extend((packed, x, y))
    nbytes = qg_batch_worklist_bytes(len(entries))
    if worklist is None:
        dev = entries[0][0].device if entries else None
        worklist = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    plan = BatchPlan()
    _check(raw().qg_batch_plan_build(fmt, M, len(entries), descs, out_dtype, kernel, _ptr(worklist),
                                     worklist.numel(), C.byref(plan), _stream(stream)),
           "qg_batch_plan_build")
    return Plan(plan, worklist, keep)


def qg_plain_read(buf, sink, grid: int, stream=None):
    """Read the whole device tensor `buf` once (plain streaming loads); the
    XOR of each workgroup's words lands in sink[j] (int32 device tensor of at
    least `grid` elements)."""
    nbytes = buf.numel() * buf.element_size()
    if sink.numel() < grid:
        raise ValueError("sink holds %d words, grid is %d" % (sink.numel(), grid))
    _check(raw().qg_plain_read(_ptr(buf), nbytes, _ptr(sink), grid, _stream(stream)),
           "qg_plain_read")


def qg_batch_run(plan: Plan, stream=None):
    _check(raw().qg_batch_run(C.byref(plan.plan), _stream(stream)), "qg_batch_run")
