"""C-ABI boundary tests that need no GPU.

The library must load, export every function include/qgemv.h declares, and
reject invalid calls with the documented status before any HIP call (every
call below fails validation, or is an empty problem that enqueues nothing,
so no pointer is ever dereferenced).
"""
import ctypes as C
import os
import re

import pytest

from conftest import ROOT, gpu_visible
import quantized_weight_decode_dequant_amd as pkg
from quantized_weight_decode_dequant_amd import _lib as L

HEADER = os.path.join(ROOT, "include", "qgemv.h")
A = 0x10000  # an aligned fake device address: only used in calls that fail validation
SZ = C.c_size_t

# The calls below pass fake device addresses and rely on the library
# rejecting them before any HIP call.  Where a GPU is visible, a regression
# of one host check would launch a kernel on such an address, so there this
# module runs only in a child process with every GPU hidden
# (test_zz_boundary_isolated.py), where a launch fails with QG_EHIP instead.
CHILD = os.environ.get("QG_BOUNDARY_CHILD") == "1"
if CHILD:
    assert not gpu_visible(), "the boundary child process still sees a GPU"
pytestmark = pytest.mark.skipif(
    not CHILD and gpu_visible(),
    reason="a GPU is visible: runs in a child process with every GPU hidden "
           "(test_zz_boundary_isolated.py)")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\**\s*([A-Za-z_]\w*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_library_loads_and_exports_every_declared_symbol():
    lib = pkg.raw()
    declared = declared_functions()
    assert set(declared) == set(L.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.qg_version() >= 100


def test_status_strings():
    for st in range(0, -8, -1):
        s = pkg.status_string(st)
        assert s.startswith("QG_")
    assert pkg.status_string(-99) == "unknown qg_status"


def size_query(fmt, rows, K):
    n = SZ(123)
    st = pkg.raw().qgemv_pack(fmt, rows, K, None, None, None, None, C.byref(n), None)
    return st, n.value


def test_pack_size_query():
    assert size_query(L.FMT_Q4_ASYM_G64, 16, 128) == (0, 1152)
    assert size_query(L.FMT_Q4_ASYM_G64, 17, 128) == (0, 2304)
    assert size_query(L.FMT_Q4_ASYM_G64, 16, 192) == (0, 2304)
    assert size_query(L.FMT_Q4_ASYM_G64, 4096, 4096) == (0, 4096 * 4096 * 9 // 16)
    assert size_query(L.FMT_Q8_SYM_G32, 16, 128) == (0, 2176)
    assert size_query(L.FMT_Q8_SYM_G32, 16, 32) == (0, 2176)
    assert size_query(L.FMT_MXFP4_G32, 16, 256) == (0, 2176)
    assert size_query(L.FMT_MXFP4_G32, 2048, 7168) == (0, 2048 * 7168 * 17 // 32)
    assert size_query(L.FMT_Q4_ASYM_G64, 0, 64) == (0, 0)
    assert size_query(L.FMT_Q4_ASYM_G64, 16, 96)[0] == L.QG_ESHAPE
    assert size_query(L.FMT_Q8_SYM_G32, 16, 48)[0] == L.QG_ESHAPE
    assert size_query(L.FMT_Q4_ASYM_G64, 16, 0)[0] == L.QG_ESHAPE
    assert size_query(L.FMT_Q4_ASYM_G64, -1, 64)[0] == L.QG_ESHAPE
    assert size_query(7, 16, 64)[0] == L.QG_EINVAL
    assert pkg.raw().qgemv_pack(1, 16, 64, None, None, None, None, None, None) == L.QG_EINVAL


def test_pack_argument_errors():
    lib = pkg.raw()
    n = SZ(1 << 20)
    # Q4 needs biases, Q8 must not have them
    assert lib.qgemv_pack(1, 16, 64, A, A, None, A, C.byref(n), None) == L.QG_EINVAL
    assert lib.qgemv_pack(2, 16, 64, A, A, A, A, C.byref(n), None) == L.QG_EINVAL
    assert lib.qgemv_pack(1, 16, 64, None, A, A, A, C.byref(n), None) == L.QG_EINVAL
    small = SZ(100)
    assert lib.qgemv_pack(1, 16, 64, A, A, A, A, C.byref(small), None) == L.QG_ESIZE
    assert small.value == 1152
    assert lib.qgemv_pack(1, 16, 64, A, A, A, A + 8, C.byref(n), None) == L.QG_EALIGN
    assert lib.qgemv_pack(1, 16, 64, A + 4, A, A, A, C.byref(n), None) == L.QG_EALIGN
    # empty problem: nothing to do
    z = SZ(0)
    assert lib.qgemv_pack(1, 0, 64, A, A, A, A, C.byref(z), None) == L.QG_OK


def test_gemv_validation():
    lib = pkg.raw()
    q4 = L.FMT_Q4_ASYM_G64
    nb = 1152 * 2  # N = 32, K = 128
    assert lib.qgemv_run(q4, A, nb, 32, 128, A, A, 7, None) == L.QG_EINVAL
    assert lib.qgemv_run(9, A, nb, 32, 128, A, A, 0, None) == L.QG_EINVAL
    assert lib.qgemv_run(L.FMT_Q8_SYM_G32, A, nb, 32, 128, A, A, 0, None) == L.QG_EUNSUPPORTED
    assert lib.qgemv_run(q4, A, nb, 32, 128, A, A, L.OUT_I32_GROUPS, None) == L.QG_EUNSUPPORTED
    assert lib.qgemv_run(q4, A, nb, 32, 100, A, A, 0, None) == L.QG_ESHAPE
    assert lib.qgemv_run(q4, A, nb + 1, 32, 128, A, A, 0, None) == L.QG_ESIZE
    assert lib.qgemv_run(q4, None, nb, 32, 128, A, A, 0, None) == L.QG_EINVAL
    assert lib.qgemv_run(q4, A, nb, 32, 128, None, A, 0, None) == L.QG_EINVAL
    assert lib.qgemv_run(q4, A + 2, nb, 32, 128, A, A, 0, None) == L.QG_EALIGN
    assert lib.qgemv_run(q4, A, nb, 32, 128, A + 8, A, 0, None) == L.QG_EALIGN
    assert lib.qgemv_run(q4, A, nb, 32, 128, A, A + 1, 0, None) == L.QG_EALIGN
    assert lib.qgemv_run(q4, A, nb, 32, 128, A, A + 2, L.OUT_F32, None) == L.QG_EALIGN
    kbig = 24576 + 64
    assert lib.qgemv_run(q4, A, pkg.packed_bytes(q4, 32, kbig), 32, kbig, A, A, 0, None) == L.QG_ESHAPE
    # N = 0 is an empty problem: OK, nothing enqueued
    assert lib.qgemv_run(q4, A, 0, 0, 128, A, A, 0, None) == L.QG_OK


def test_skinny_validation():
    lib = pkg.raw()
    q4, q8 = L.FMT_Q4_ASYM_G64, L.FMT_Q8_SYM_G32
    nb4 = pkg.packed_bytes(q4, 32, 128)
    nb8 = pkg.packed_bytes(q8, 32, 128)
    assert lib.qgemm_skinny_run(q4, A, nb4, 33, 32, 128, A, None, A, 0, None) == L.QG_ESHAPE
    assert lib.qgemm_skinny_run(q4, A, nb4, -1, 32, 128, A, None, A, 0, None) == L.QG_ESHAPE
    assert lib.qgemm_skinny_run(L.FMT_MXFP4_G32, A, nb4, 4, 32, 128, A, None, A, 0, None) == L.QG_EUNSUPPORTED
    assert lib.qgemm_skinny_run(q4, A, nb4, 4, 32, 128, A, None, A, L.OUT_I32_GROUPS, None) == L.QG_EUNSUPPORTED
    assert lib.qgemm_skinny_run(q4, A, nb4, 4, 32, 128, A, A, A, 0, None) == L.QG_EINVAL
    assert lib.qgemm_skinny_run(q8, A, nb8, 4, 32, 128, A, None, A, 0, None) == L.QG_EINVAL
    assert lib.qgemm_skinny_run(q8, A, nb8 - 16, 4, 32, 128, A, A, A, 0, None) == L.QG_ESIZE
    assert lib.qgemm_skinny_run(q8, A, nb8, 4, 32, 128, A + 4, A, A, 0, None) == L.QG_EALIGN
    assert lib.qgemm_skinny_run(q8, A, nb8, 4, 32, 128, A, A + 2, A, 0, None) == L.QG_EALIGN
    assert lib.qgemm_skinny_run(q8, A, nb8, 4, 32, 128, A, A, A + 2, L.OUT_I32_GROUPS, None) == L.QG_EALIGN
    assert lib.qgemm_skinny_run(q8, A, nb8, 0, 32, 128, A, A, A, 0, None) == L.QG_OK


def test_hadamard_validation():
    lib = pkg.raw()
    assert lib.hadamard32_quant_run(A, A, 4, 48, A, A, None) == L.QG_ESHAPE
    assert lib.hadamard32_quant_run(A, A, 4, 0, A, A, None) == L.QG_ESHAPE
    assert lib.hadamard32_quant_run(None, A, 4, 64, A, A, None) == L.QG_EINVAL
    assert lib.hadamard32_quant_run(A, None, 4, 64, A, A, None) == L.QG_EINVAL
    assert lib.hadamard32_quant_run(A + 2, A, 4, 64, A, A, None) == L.QG_EALIGN
    assert lib.hadamard32_quant_run(A, A, 4, 64, A + 1, A, None) == L.QG_EALIGN
    assert lib.hadamard32_quant_run(A, A + 1, 4, 64, A, A, None) == L.QG_EALIGN
    assert lib.hadamard32_quant_run(A, A, 0, 64, A, A, None) == L.QG_OK


def test_plain_read_validation():
    lib = pkg.raw()
    assert lib.qg_plain_read(None, 64, A, 4, None) == L.QG_EINVAL
    assert lib.qg_plain_read(A, 64, None, 4, None) == L.QG_EINVAL
    assert lib.qg_plain_read(A, 65, A, 4, None) == L.QG_ESHAPE
    assert lib.qg_plain_read(A, 64, A, 0, None) == L.QG_ESHAPE
    assert lib.qg_plain_read(A, 64, A, 65537, None) == L.QG_ESHAPE
    assert lib.qg_plain_read(A + 8, 64, A, 4, None) == L.QG_EALIGN
    assert lib.qg_plain_read(A, 64, A + 2, 4, None) == L.QG_EALIGN
    assert lib.qg_plain_read(A, 0, A, 4, None) == L.QG_OK


def test_moe_validation():
    lib = pkg.raw()
    E, H, F, k = 8, 256, 512, 2
    bg = pkg.packed_bytes(L.FMT_MXFP4_G32, E * F, H)
    bd = pkg.packed_bytes(L.FMT_MXFP4_G32, E * H, F)
    ws = pkg.moe_workspace_bytes(k, H, F)
    assert ws == 4 * k * (H + F) + 16

    def call(**kw):
        a = dict(g=A, u=A, d=A, bg=bg, bu=bg, bd=bd, E=E, H=H, F=F, x=A, k=k, ids=A, w=A, ws=A,
                 wsb=ws, y=A, out=0)
        a.update(kw)
        return lib.moe_expert_gemv_run(a["g"], a["u"], a["d"], a["bg"], a["bu"], a["bd"], a["E"],
                                       a["H"], a["F"], a["x"], a["k"], a["ids"], a["w"], a["ws"],
                                       a["wsb"], a["y"], a["out"], None)

    assert call(out=5) == L.QG_EINVAL
    assert call(out=L.OUT_I32_GROUPS) == L.QG_EUNSUPPORTED
    assert call(k=E + 1) == L.QG_ESHAPE
    assert call(k=65) == L.QG_ESHAPE
    assert call(H=250) == L.QG_ESHAPE
    assert call(F=12288 + 32) == L.QG_ESHAPE
    assert call(E=0) == L.QG_ESHAPE
    assert call(g=None) == L.QG_EINVAL
    assert call(ids=None) == L.QG_EINVAL
    assert call(bd=bd + 16) == L.QG_ESIZE
    assert call(bg=bg - 16) == L.QG_ESIZE
    assert call(wsb=ws - 1) == L.QG_ESIZE
    assert call(ws=A + 8) == L.QG_EALIGN
    assert call(ids=A + 2) == L.QG_EALIGN
    assert call(ws=None) == L.QG_EINVAL


def test_moe_noalloc_validation():
    """The allocation-free MoE call: the checks of moe_expert_gemv_run, and
    QG_ESIZE for a layer whose workspace exceeds the library's array."""
    lib = pkg.raw()
    E, H, F, k = 8, 256, 512, 2
    bg = pkg.packed_bytes(L.FMT_MXFP4_G32, E * F, H)
    bd = pkg.packed_bytes(L.FMT_MXFP4_G32, E * H, F)

    def call(**kw):
        a = dict(g=A, u=A, d=A, bg=bg, bu=bg, bd=bd, E=E, H=H, F=F, x=A, k=k, ids=A, w=A,
                 st=A, y=A, out=0)
        a.update(kw)
        return lib.moe_expert_gemv_run_noalloc(a["g"], a["u"], a["d"], a["bg"], a["bu"], a["bd"],
                                               a["E"], a["H"], a["F"], a["x"], a["k"], a["ids"],
                                               a["w"], a["st"], a["y"], a["out"], None)

    assert call(out=5) == L.QG_EINVAL
    assert call(out=L.OUT_I32_GROUPS) == L.QG_EUNSUPPORTED
    assert call(k=E + 1) == L.QG_ESHAPE
    assert call(H=250) == L.QG_ESHAPE
    assert call(g=None) == L.QG_EINVAL
    assert call(x=None) == L.QG_EINVAL
    assert call(y=None) == L.QG_EINVAL
    assert call(ids=None) == L.QG_EINVAL
    assert call(bd=bd + 16) == L.QG_ESIZE
    assert call(x=A + 8) == L.QG_EALIGN
    assert call(st=A + 2) == L.QG_EALIGN
    assert call(y=A + 1) == L.QG_EALIGN
    # top-16 of H = 24576, F = 12288 needs 4 * 16 * 36864 + 16 bytes > 2 MiB
    E2, H2, F2, k2 = 16, 24576, 12288, 16
    assert pkg.moe_workspace_bytes(k2, H2, F2) > L.MOE_NOALLOC_SCRATCH_BYTES
    assert pkg.moe_workspace_bytes(16, 7168, 2048) <= L.MOE_NOALLOC_SCRATCH_BYTES
    bg2 = pkg.packed_bytes(L.FMT_MXFP4_G32, E2 * F2, H2)
    bd2 = pkg.packed_bytes(L.FMT_MXFP4_G32, E2 * H2, F2)
    assert call(E=E2, H=H2, F=F2, k=k2, bg=bg2, bu=bg2, bd=bd2) == L.QG_ESIZE


def test_moe_skinny_validation():
    lib = pkg.raw()
    E, H, F, k, T = 8, 256, 512, 2, 5
    bg = pkg.packed_bytes(L.FMT_MXFP4_G32, E * F, H)
    bd = pkg.packed_bytes(L.FMT_MXFP4_G32, E * H, F)
    ws = pkg.moe_skinny_workspace_bytes(T, k, H, F)
    assert ws == 4 * T * k * (H + F) + 16 + 32 * T * k

    def call(**kw):
        a = dict(g=A, u=A, d=A, bg=bg, bu=bg, bd=bd, E=E, H=H, F=F, T=T, X=A, k=k, ids=A, w=A,
                 ws=A, wsb=ws, Y=A, out=0)
        a.update(kw)
        return lib.moe_expert_skinny_run(a["g"], a["u"], a["d"], a["bg"], a["bu"], a["bd"],
                                         a["E"], a["H"], a["F"], a["T"], a["X"], a["k"],
                                         a["ids"], a["w"], a["ws"], a["wsb"], a["Y"], a["out"],
                                         None)

    assert call(out=5) == L.QG_EINVAL
    assert call(out=L.OUT_I32_GROUPS) == L.QG_EUNSUPPORTED
    assert call(T=0) == L.QG_ESHAPE
    assert call(T=33) == L.QG_ESHAPE
    assert call(k=E + 1) == L.QG_ESHAPE
    assert call(E=65, k=65, T=32) == L.QG_ESHAPE  # top_k above 64
    assert call(H=250) == L.QG_ESHAPE
    assert call(F=12288 + 32) == L.QG_ESHAPE
    assert call(X=None) == L.QG_EINVAL
    assert call(Y=None) == L.QG_EINVAL
    assert call(w=None) == L.QG_EINVAL
    assert call(bg=bg + 16) == L.QG_ESIZE
    assert call(wsb=ws - 1) == L.QG_ESIZE
    assert call(X=A + 8) == L.QG_EALIGN
    assert call(Y=A + 1) == L.QG_EALIGN
    assert call(out=L.OUT_F32, Y=A + 2) == L.QG_EALIGN
    assert call(ws=A + 8) == L.QG_EALIGN


def test_q8row_validation():
    lib = pkg.raw()
    f = L.FMT_Q8_ROW
    n = C.c_size_t(0)
    assert lib.qgemv_pack(f, 40, 288, None, None, None, None, C.byref(n), None) == L.QG_OK
    assert n.value == 3 * (3 * 2048 + 64)  # 3 rowblocks of 3 tiles and 64 B of row scales
    cap = C.c_size_t(n.value)
    assert lib.qgemv_pack(f, 40, 272, A, A, None, A, C.byref(cap), None) == L.QG_ESHAPE
    assert lib.qgemv_pack(f, 40, 288, A, A, A, A, C.byref(cap), None) == L.QG_EINVAL  # no biases
    assert lib.qgemv_pack(f, 40, 288, A, A + 2, None, A, C.byref(cap), None) == L.QG_EALIGN
    assert lib.qgemv_run(f, A, n.value, 40, 288, A, A, 2, None) == L.QG_EUNSUPPORTED
    assert lib.qgemv_run(f, A, n.value + 1, 40, 288, A, A, 0, None) == L.QG_ESIZE
    assert lib.qgemv_run(f, A, n.value, 40, 288, A + 8, A, 0, None) == L.QG_EALIGN
    assert lib.qgemm_skinny_run(f, A, n.value, 2, 40, 288, A, None, A, 0, None) == L.QG_EUNSUPPORTED


def test_affine_validation():
    lib = pkg.raw()
    f = L.affine_format(3, 32, True)
    assert f == 0x100 | (3 << 4) | (0 << 2) | 1
    n = C.c_size_t(0)
    assert lib.qgemv_pack(f, 40, 96, None, None, None, None, C.byref(n), None) == L.QG_OK
    assert n.value == 3 * (256 * 3 + 16 * 4 * 4)  # 3 rowblocks x 1 tile
    for bad in (L.affine_format(7, 32), L.affine_format(1, 32), L.affine_format(4, 16),
                L.affine_format(4, 256), 0x244, 0x100 | (4 << 4) | (3 << 2)):
        assert lib.qgemv_pack(bad, 40, 96, None, None, None, None, C.byref(n), None) == L.QG_EINVAL
    f64 = L.affine_format(4, 64)
    assert lib.qgemv_pack(f64, 40, 96, None, None, None, None, C.byref(n), None) == L.QG_ESHAPE
    need = pkg.packed_bytes(f, 40, 96)
    cap = C.c_size_t(need)
    assert lib.qgemv_pack(f, 40, 96, A, A, None, A, C.byref(cap), None) == L.QG_EINVAL  # biases
    assert lib.qgemv_run(f, A, need + 16, 40, 96, A, A, 0, None) == L.QG_ESIZE
    assert lib.qgemv_run(f, A, need, 40, 96, A + 4, A, 0, None) == L.QG_EALIGN
    # the skinny product takes affine codes; every call below fails validation
    assert lib.qgemm_skinny_run(f, A, need, 2, 40, 96, A, A, A, 0, None) == L.QG_EINVAL  # scales
    assert lib.qgemm_skinny_run(f, A, need, 2, 40, 96, A, None, A, 2, None) == L.QG_EUNSUPPORTED
    assert lib.qgemm_skinny_run(f, A, need, 33, 40, 96, A, None, A, 0, None) == L.QG_ESHAPE
    assert lib.qgemm_skinny_run(f, A, need + 16, 2, 40, 96, A, None, A, 0, None) == L.QG_ESIZE
    assert lib.qgemm_skinny_run(f, A, need, 2, 40, 96, A + 8, None, A, 0, None) == L.QG_EALIGN


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        pkg.qgemv_run(L.FMT_Q4_ASYM_G64, torch.zeros(1152, dtype=torch.uint8), 16, 128,
                      torch.zeros(128, dtype=torch.bfloat16), y=torch.zeros(16))


def test_batch_validation():
    """Every call fails validation before touching the device (no plan here is
    ever well-formed enough to launch)."""
    lib = pkg.raw()
    q4 = L.FMT_Q4_ASYM_G64
    n = 3
    wl = pkg.qg_batch_worklist_bytes(n)
    assert wl == 64 + 48 * n + 8 * 4097
    good = dict(packed=A, packed_bytes=pkg.packed_bytes(q4, 64, 256), N=64, K=256, x=A, y=A)

    def descs(**over):
        arr = (L.GemvDesc * n)()
        for i in range(n):
            d = dict(good)
            if i == 1:
                d.update(over)
            for k, v in d.items():
                setattr(arr[i], k, v)
        return arr

    plan = L.BatchPlan()

    def build(fmt=q4, M=1, count=n, arr=None, out=0, kernel=0, wl_ptr=A, wl_bytes=wl,
              plan_ptr=True):
        arr = descs() if arr is None else arr
        return lib.qg_batch_plan_build(fmt, M, count, arr, out, kernel, wl_ptr, wl_bytes,
                                       C.byref(plan) if plan_ptr else None, None)

    assert build(plan_ptr=False) == L.QG_EINVAL
    assert build(wl_ptr=None) == L.QG_EINVAL
    assert build(out=5) == L.QG_EINVAL
    assert build(out=L.OUT_I32_GROUPS) == L.QG_EUNSUPPORTED
    assert build(fmt=9) == L.QG_EINVAL
    assert build(fmt=L.FMT_Q8_SYM_G32) == L.QG_EUNSUPPORTED
    assert build(M=0) == L.QG_ESHAPE
    assert build(M=33) == L.QG_ESHAPE
    assert build(kernel=3) == L.QG_EINVAL
    assert build(kernel=-1) == L.QG_EINVAL
    assert build(M=5, kernel=L.KERNEL_VALU) == L.QG_EUNSUPPORTED
    assert build(count=0) == L.QG_ESHAPE
    assert build(wl_bytes=wl - 1) == L.QG_ESIZE
    assert build(wl_ptr=A + 4) == L.QG_EALIGN
    assert build(arr=descs(K=100)) == L.QG_ESHAPE
    assert build(arr=descs(N=0, packed_bytes=0)) == L.QG_ESHAPE
    assert build(arr=descs(K=24576 + 64, packed_bytes=pkg.packed_bytes(q4, 64, 24576 + 64))) == L.QG_ESHAPE
    assert build(arr=descs(packed_bytes=123)) == L.QG_ESIZE
    assert build(arr=descs(x=None)) == L.QG_EINVAL
    assert build(arr=descs(x=A + 2)) == L.QG_EALIGN
    assert build(arr=descs(y=A + 1)) == L.QG_EALIGN
    assert build(arr=descs(y=A + 2), out=L.OUT_F32) == L.QG_EALIGN
    # affine products: the GEMV kernel at M = 1, the MFMA kernel for more rows;
    # every descriptor of the plan's format
    aff = pkg.affine_format(3, 32, False)
    assert build(fmt=aff, kernel=L.KERNEL_MFMA) == L.QG_EUNSUPPORTED
    assert build(fmt=aff, M=2, kernel=L.KERNEL_VALU) == L.QG_EUNSUPPORTED
    assert build(fmt=aff, M=16, kernel=L.KERNEL_VALU) == L.QG_EUNSUPPORTED
    assert build(fmt=aff) == L.QG_ESIZE  # the descriptors are sized as Q4
    assert build(fmt=aff, M=2) == L.QG_ESIZE
    assert build(fmt=aff, M=32, kernel=L.KERNEL_MFMA) == L.QG_ESIZE
    # int8 row-scale GEMVs: one activation row, the GEMV kernel only
    q8r = L.FMT_Q8_ROW
    assert build(fmt=q8r, M=2) == L.QG_EUNSUPPORTED
    assert build(fmt=q8r, kernel=L.KERNEL_MFMA) == L.QG_EUNSUPPORTED
    assert build(fmt=q8r) == L.QG_ESIZE  # the descriptors are sized as Q4
    q4_bytes = good["packed_bytes"]
    good["packed_bytes"] = pkg.packed_bytes(q8r, 64, 256)
    assert build(fmt=q8r, arr=descs(K=48)) == L.QG_ESHAPE
    assert build(fmt=q8r, arr=descs(K=24576 + 32,
                                     packed_bytes=pkg.packed_bytes(q8r, 64, 24576 + 32))) == L.QG_ESHAPE
    good["packed_bytes"] = q4_bytes
    good["packed_bytes"] = pkg.packed_bytes(aff, 64, 256)
    assert build(fmt=aff, arr=descs(K=48)) == L.QG_ESHAPE
    assert build(fmt=aff, arr=descs(K=24576 + 32)) == L.QG_ESHAPE
    assert build(fmt=aff, arr=descs(packed_bytes=9216)) == L.QG_ESIZE
    assert build(fmt=aff, M=2, kernel=L.KERNEL_VALU) == L.QG_EUNSUPPORTED
    assert build(fmt=pkg.affine_format(7, 32, False)) == L.QG_EINVAL
    # malformed plans are refused before any launch
    assert lib.qg_batch_run(None, None) == L.QG_EINVAL
    bad = L.BatchPlan()
    assert lib.qg_batch_run(C.byref(bad), None) == L.QG_EINVAL
    bad.fmt, bad.M, bad.count, bad.grid, bad.kmax = q4, 1, 3, 4, 256
    bad.worklist, bad.worklist_bytes = A, wl
    bad.kernel = L.KERNEL_AUTO
    assert lib.qg_batch_run(C.byref(bad), None) == L.QG_EINVAL  # kernel not chosen
    bad.kernel, bad.M = L.KERNEL_VALU, 5
    assert lib.qg_batch_run(C.byref(bad), None) == L.QG_EINVAL  # VALU kernel past 4 rows
    bad.kernel, bad.M, bad.grid = L.KERNEL_VALU, 1, 0
    assert lib.qg_batch_run(C.byref(bad), None) == L.QG_EINVAL  # grid 0
    bad.grid = 5000
    assert lib.qg_batch_run(C.byref(bad), None) == L.QG_EINVAL  # grid > max
    bad.grid, bad.worklist_bytes = 4, wl - 8
    assert lib.qg_batch_run(C.byref(bad), None) == L.QG_EINVAL  # work list too small
    bad.fmt, bad.worklist_bytes, bad.M = aff, wl, 2
    assert lib.qg_batch_run(C.byref(bad), None) == L.QG_EINVAL  # affine GEMV kernel past one row
    bad.M, bad.kernel = 1, L.KERNEL_MFMA
    assert lib.qg_batch_run(C.byref(bad), None) == L.QG_EINVAL  # affine MFMA kernel at one row
    bad.fmt = L.FMT_Q8_ROW
    assert lib.qg_batch_run(C.byref(bad), None) == L.QG_EINVAL  # int8 rows on the MFMA family
    bad.kernel, bad.M = L.KERNEL_VALU, 2
    assert lib.qg_batch_run(C.byref(bad), None) == L.QG_EINVAL  # int8 rows past one row
    bad.fmt, bad.M, bad.kernel = aff, 1, L.KERNEL_MFMA
    bad.kernel, bad.kmax = L.KERNEL_VALU, 16
    assert lib.qg_batch_run(C.byref(bad), None) == L.QG_EINVAL  # K below one group
