"""numpy front end of the plain C oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``.  The product never imports it.

The C library is built with gcc -O2, no fast-math and no FP contraction, so
every double operation is the IEEE operation the source states.  ``build()``
compiles it; the loader builds it on first use if the shared object is absent.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
          "-Wall", "-Wextra"]


def build() -> str:
    """Compile oracle.c into liboracle.so (always recompiles)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            lib = C.CDLL(_LIB)
            i64, p = C.c_int64, C.c_void_p
            sigs = {
                "oracle_f16_to_f64": ([C.c_uint16], C.c_double),
                "oracle_bf16_to_f64": ([C.c_uint16], C.c_double),
                "oracle_e2m1": ([C.c_uint], C.c_double),
                "oracle_e8m0": ([C.c_uint], C.c_double),
                "oracle_h32": ([C.c_int, C.c_int], C.c_int),
                "oracle_silu": ([C.c_double], C.c_double),
                "oracle_q4_gemm": ([i64, i64, i64, p, p, p, p, p], None),
                "oracle_hadamard32": ([i64, i64, p, p, p], None),
                "oracle_quant_rows_int8": ([i64, i64, p, p, p], None),
                "oracle_had32_quant": ([i64, i64, p, p, p, p, p], None),
                "oracle_q8_group_acc": ([i64, i64, i64, p, p, p], None),
                "oracle_q8_gemm": ([i64, i64, i64, p, p, p, p, p], None),
                "oracle_mxfp4_gemv": ([i64, i64, p, p, p, p], None),
                "oracle_mxfp4_gemv_f64": ([i64, i64, p, p, p, p], None),
                "oracle_q8row_gemv": ([i64, i64, p, p, p, p], None),
                "oracle_affine_gemv": ([i64, i64, i64, C.c_int, p, p, p, p, p], None),
                "oracle_moe": ([i64, i64, i64, p, p, p, p, p, p, p, i64, p, p, p, p, p, p, p],
                               None),
            }
            for name, (args, res) in sigs.items():
                f = getattr(lib, name)
                f.argtypes = args
                f.restype = res
            _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(C.c_void_p)


# ------------------------------------------------------------------ scalars
def f16_to_f64(h: int) -> float:
    return _load().oracle_f16_to_f64(int(h))


def bf16_to_f64(b: int) -> float:
    return _load().oracle_bf16_to_f64(int(b))


def e2m1(code: int) -> float:
    return _load().oracle_e2m1(int(code))


def e8m0(e: int) -> float:
    return _load().oracle_e8m0(int(e))


def h32(i: int, j: int) -> int:
    return _load().oracle_h32(int(i), int(j))


def silu(a: float) -> float:
    return _load().oracle_silu(float(a))


# ------------------------------------------------------------------ Q4 g64
def q4_gemm(codes, scales, biases, X) -> np.ndarray:
    """Y [M, N] (float64) = X [M, K] (bf16 bits) . W^T, W = Q4 g64 [N, K]."""
    codes, pc = _c(codes, np.uint32)
    scales, ps = _c(scales, np.uint16)
    biases, pb = _c(biases, np.uint16)
    X = np.atleast_2d(X)
    X, px = _c(X, np.uint16)
    N, K = codes.shape[0], codes.shape[1] * 8
    M = X.shape[0]
    assert X.shape[1] == K and scales.shape == (N, K // 64) and biases.shape == (N, K // 64)
    Y = np.empty((M, N), dtype=np.float64)
    _load().oracle_q4_gemm(M, N, K, pc, ps, pb, px, Y.ctypes.data_as(C.c_void_p))
    return Y


# ------------------------------------------------------- Hadamard + int8 quant
def hadamard32(X, signs) -> np.ndarray:
    X = np.atleast_2d(X)
    X, px = _c(X, np.uint16)
    signs, pd = _c(signs, np.int8)
    M, K = X.shape
    assert K % 32 == 0 and signs.shape == (K,)
    Z = np.empty((M, K), dtype=np.float64)
    _load().oracle_hadamard32(M, K, px, pd, Z.ctypes.data_as(C.c_void_p))
    return Z


def quant_rows_int8(Z):
    Z = np.atleast_2d(Z)
    Z, pz = _c(Z, np.float64)
    M, K = Z.shape
    Q = np.empty((M, K), dtype=np.int8)
    sx = np.empty(M, dtype=np.float32)
    _load().oracle_quant_rows_int8(M, K, pz, Q.ctypes.data_as(C.c_void_p),
                                   sx.ctypes.data_as(C.c_void_p))
    return Q, sx


def had32_quant(X, signs):
    """(Xq int8 [M, K], sx float32 [M]) for bf16 X [M, K] and +-1 signs [K]."""
    X = np.atleast_2d(X)
    X, px = _c(X, np.uint16)
    signs, pd = _c(signs, np.int8)
    M, K = X.shape
    assert K % 32 == 0 and signs.shape == (K,)
    Z = np.empty((M, K), dtype=np.float64)
    Q = np.empty((M, K), dtype=np.int8)
    sx = np.empty(M, dtype=np.float32)
    _load().oracle_had32_quant(M, K, px, pd, Z.ctypes.data_as(C.c_void_p),
                               Q.ctypes.data_as(C.c_void_p), sx.ctypes.data_as(C.c_void_p))
    return Q, sx


# ------------------------------------------------------------------ Q8 g32
def q8_group_acc(qw, qx) -> np.ndarray:
    qw, pw = _c(qw, np.int8)
    qx = np.atleast_2d(qx)
    qx, px = _c(qx, np.int8)
    N, K = qw.shape
    M = qx.shape[0]
    assert qx.shape[1] == K and K % 32 == 0
    acc = np.empty((M, N, K // 32), dtype=np.int32)
    _load().oracle_q8_group_acc(M, N, K, pw, px, acc.ctypes.data_as(C.c_void_p))
    return acc


def q8_gemm(qw, sw, qx, sx) -> np.ndarray:
    qw, pw = _c(qw, np.int8)
    sw, psw = _c(sw, np.uint16)
    qx = np.atleast_2d(qx)
    qx, px = _c(qx, np.int8)
    sx, psx = _c(np.atleast_1d(sx), np.float32)
    N, K = qw.shape
    M = qx.shape[0]
    assert qx.shape[1] == K and sw.shape == (N, K // 32) and sx.shape == (M,)
    Y = np.empty((M, N), dtype=np.float64)
    _load().oracle_q8_gemm(M, N, K, pw, psw, px, psx, Y.ctypes.data_as(C.c_void_p))
    return Y


# ------------------------------------------------------------------ MXFP4
def mxfp4_gemv(codes, scales, x) -> np.ndarray:
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(scales, np.uint8)
    N, K = codes.shape[0], codes.shape[1] * 2
    x = np.asarray(x)
    y = np.empty(N, dtype=np.float64)
    if x.dtype == np.float64:
        x, px = _c(x, np.float64)
        assert x.shape == (K,)
        _load().oracle_mxfp4_gemv_f64(N, K, pc, ps, px, y.ctypes.data_as(C.c_void_p))
    else:
        x, px = _c(x, np.uint16)
        assert x.shape == (K,)
        _load().oracle_mxfp4_gemv(N, K, pc, ps, px, y.ctypes.data_as(C.c_void_p))
    return y


def q8row_gemv(codes, scales, x):
    """y [N] (float64) for weight-only int8: codes int8 [N, K], scales float32
    [N] (one per row), x bf16 bits [K]."""
    codes, pc = _c(codes, np.int8)
    scales, ps = _c(scales, np.float32)
    x, px = _c(x, np.uint16)
    N, K = codes.shape
    assert scales.shape == (N,) and x.shape == (K,)
    y = np.empty(N)
    _load().oracle_q8row_gemv(N, K, pc, ps, px, y.ctypes.data_as(C.c_void_p))
    return y


def affine_gemv(codes, scales, biases, x, group: int, bf16_scales: bool):
    """y [N] (float64) for the affine family: codes uint8 [N, K] (one code
    per byte), scales and biases fp16 or bf16 bits [N, K/group], x bf16 bits
    [K]."""
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(scales, np.uint16)
    biases, pb = _c(biases, np.uint16)
    x, px = _c(x, np.uint16)
    N, K = codes.shape
    assert K % group == 0 and scales.shape == (N, K // group) and biases.shape == scales.shape
    assert x.shape == (K,)
    y = np.empty(N)
    _load().oracle_affine_gemv(N, K, group, 1 if bf16_scales else 0, pc, ps, pb, px,
                               y.ctypes.data_as(C.c_void_p))
    return y


def affine_gemm(codes, scales, biases, X, group: int, bf16_scales: bool):
    """Y [M, N] (float64): the affine-family product for each row of X (bf16
    bits [M, K]), row by row through ``affine_gemv``."""
    X = np.asarray(X, dtype=np.uint16)
    return np.stack([affine_gemv(codes, scales, biases, X[m], group, bf16_scales)
                     for m in range(X.shape[0])])


def moe(gate_codes, gate_scales, up_codes, up_scales, down_codes, down_scales, x, ids, w):
    """y [H] (float64) for one token through the routed experts.

    gate/up codes [E, F, H/2], scales [E, F, H/32]; down codes [E, H, F/2],
    scales [E, H, F/32]; x bf16 bits [H]; ids int32 [top_k]; w float32 [top_k]."""
    gc, pgc = _c(gate_codes, np.uint8)
    gs, pgs = _c(gate_scales, np.uint8)
    uc, puc = _c(up_codes, np.uint8)
    us, pus = _c(up_scales, np.uint8)
    dc, pdc = _c(down_codes, np.uint8)
    ds, pds = _c(down_scales, np.uint8)
    x, px = _c(x, np.uint16)
    ids, pid = _c(ids, np.int32)
    w, pw = _c(w, np.float32)
    E, F, H = gc.shape[0], gc.shape[1], gc.shape[2] * 2
    assert uc.shape == gc.shape and dc.shape == (E, H, F // 2)
    assert gs.shape == (E, F, H // 32) and us.shape == gs.shape and ds.shape == (E, H, F // 32)
    assert x.shape == (H,) and ids.shape == w.shape
    top_k = ids.shape[0]
    g = np.empty(F)
    u = np.empty(F)
    h = np.empty(F)
    d = np.empty(H)
    y = np.empty(H)
    vp = lambda a: a.ctypes.data_as(C.c_void_p)  # noqa: E731
    _load().oracle_moe(E, H, F, pgc, pgs, puc, pus, pdc, pds, px, top_k, pid, pw,
                       vp(g), vp(u), vp(h), vp(d), vp(y))
    return y


def moe_positions(gate_codes, gate_scales, up_codes, up_scales, down_codes, down_scales, X, ids,
                  w):
    """Y [T, H] (float64): T positions through the routed experts, each with
    its own router output.  The positions are independent, so row t is the
    single-token layer (``moe``) applied to X[t], ids[t], w[t].

    X bf16 bits [T, H]; ids int32 [T, top_k]; w float32 [T, top_k]."""
    X = np.asarray(X, dtype=np.uint16)
    ids = np.asarray(ids, dtype=np.int32)
    w = np.asarray(w, dtype=np.float32)
    assert X.ndim == 2 and ids.shape == w.shape and ids.shape[0] == X.shape[0]
    return np.stack([moe(gate_codes, gate_scales, up_codes, up_scales, down_codes, down_scales,
                         X[t], ids[t], w[t]) for t in range(X.shape[0])])
