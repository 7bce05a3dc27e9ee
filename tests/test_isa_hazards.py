"""The built gfx950 code keeps its VALU writes clear of the MFMAs around them.

Two rules, both of which the compiler keeps for its own instructions but not
for an instruction written in inline asm, which its hazard checks do not see
as a VALU write:
  - an MFMA that reads a VGPR fewer than 2 wait states after a VALU wrote it
    reads the old value;
  - a VALU write to a VGPR that an MFMA issued before it has yet to write (a
    16x16 MFMA writes its result 8 passes after issue) is overwritten by the
    MFMA's result.
Either gives wrong sums without any error.  This test disassembles the
library built here (its device code objects, extracted from the host
library's fat binary) and checks every MFMA against both rules; the scanners
are checked on planted snippets; and the kernel sources hold no asm statement
with an instruction in it (only empty ones, which make a value opaque)."""
import os
import re
import struct
import subprocess
import tempfile

import pytest

from conftest import ROOT

LIB = os.path.join(ROOT, "quantized_weight_decode_dequant_amd", "libqgemv.so")
LLVM = "/opt/rocm/llvm/bin"
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
MIN_WAIT_STATES = 2
CSRC = os.path.join(ROOT, "quantized_weight_decode_dequant_amd", "csrc")


def mfma_result_passes(opcode):
    """Wait states before a VALU may write a destination VGPR of the MFMA
    (its passes): 8 for the 16x16 shapes, 16 for 32x32, 2 for 4x4."""
    if "_32x32x" in opcode:
        return 16
    if "_16x16x" in opcode:
        return 8
    if "_4x4x" in opcode:
        return 2
    return 16


def _vgprs(operand_text):
    regs = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", operand_text):
        if m.group(3):
            regs.add(int(m.group(3)))
        else:
            regs.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return regs


def mfma_hazards(lines, min_wait=MIN_WAIT_STATES):
    """(wait states, writer, mfma) for every VALU write of an MFMA source VGPR
    fewer than min_wait wait states before the MFMA.  lines: instructions in
    program order, None at labels (the scan stops there and at branches);
    s_nop n counts n + 1 wait states, any other instruction one."""
    found = []
    for j, ins in enumerate(lines):
        if not ins or not ins.startswith("v_mfma"):
            continue
        srcs = _vgprs(",".join(ins.split(None, 1)[1].split(",")[1:]))
        waits, k = 0, j - 1
        while k >= 0 and waits < min_wait:
            prev = lines[k]
            if prev is None or prev.startswith(("s_cbranch", "s_branch", "s_setpc")):
                break
            if prev.startswith("s_nop"):
                waits += int(prev.split()[1], 0) + 1
                k -= 1
                continue
            if prev.startswith("v_") and not prev.startswith("v_mfma"):
                parts = prev.split(None, 1)
                if len(parts) > 1 and _vgprs(parts[1].split(",")[0]) & srcs:
                    found.append((waits, prev, ins))
                    break
            waits += 1
            k -= 1
    return found


def mfma_result_hazards(lines):
    """(wait states, writer, mfma) for every non-MFMA VALU write of a VGPR
    that an earlier MFMA writes, before that MFMA's passes have elapsed."""
    found = []
    for j, ins in enumerate(lines):
        if not ins or not ins.startswith("v_mfma"):
            continue
        need = mfma_result_passes(ins.split()[0])
        dst = _vgprs(ins.split(None, 1)[1].split(",")[0])
        waits, k = 0, j + 1
        while k < len(lines) and waits < need:
            nxt = lines[k]
            if nxt is None or nxt.startswith(("s_cbranch", "s_branch", "s_setpc")):
                break
            if nxt.startswith("s_nop"):
                waits += int(nxt.split()[1], 0) + 1
                k += 1
                continue
            if nxt.startswith("v_"):
                parts = nxt.split(None, 1)
                if len(parts) > 1 and _vgprs(parts[1].split(",")[0]) & dst:
                    if not nxt.startswith("v_mfma"):
                        found.append((waits, nxt, ins))
                    break
            waits += 1
            k += 1
    return found


def _instruction_lines(disassembly):
    lines = []
    for raw in disassembly.splitlines():
        t = raw.strip()
        if re.match(r"^[0-9a-f]+ <.*>:$", t) or (t.endswith(":") and " " not in t):
            lines.append(None)
            continue
        if re.match(r"^(s_|v_|buffer_|global_|ds_|flat_|scratch_)", t):
            lines.append(re.sub(r"//.*", "", t).strip())
    return lines


def _code_objects(lib):
    """The amdgcn code objects of every bundle in the library's fat binary."""
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fatbin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section",
                        ".hip_fatbin=" + fat, lib, os.path.join(d, "copy")],
                       check=True, capture_output=True)
        with open(fat, "rb") as f:
            data = f.read()
    objs = []
    for m in re.finditer(re.escape(BUNDLE_MAGIC), data):
        p = m.start()
        (n,) = struct.unpack_from("<Q", data, p + 24)
        q = p + 32
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", data, q)
            q += 24
            triple = data[q:q + tlen].decode()
            q += tlen
            if "amdgcn" in triple and "gfx950" in triple:
                objs.append(data[p + off:p + off + size])
    return objs


def test_scanner_flags_planted_hazards():
    """A VALU write one or zero wait states before the MFMA that reads it is
    flagged (as source A, B or C); two wait states, an s_nop making up the
    difference, an unrelated register or a label in between are not."""
    mfma = "v_mfma_f32_16x16x32_bf16 v[4:7], v[8:11], v[12:15], v[4:7]"
    assert len(mfma_hazards(["v_and_or_b32 v9, v1, v2, v3", mfma])) == 1
    assert len(mfma_hazards(["v_and_or_b32 v13, v1, v2, v3", "v_mov_b32 v40, 0", mfma])) == 1
    assert len(mfma_hazards(["v_add_f32 v6, v1, v2", mfma])) == 1
    assert not mfma_hazards(["v_and_or_b32 v9, v1, v2, v3", "v_mov_b32 v40, 0",
                             "v_mov_b32 v41, 0", mfma])
    assert not mfma_hazards(["v_and_or_b32 v9, v1, v2, v3", "s_nop 1", mfma])
    assert not mfma_hazards(["v_and_or_b32 v20, v1, v2, v3", mfma])
    assert not mfma_hazards(["v_and_or_b32 v9, v1, v2, v3", None, mfma])


def test_scanner_flags_planted_result_overwrites():
    """A VALU write to the destination of an MFMA issued 0..7 wait states
    before is flagged; after 8 wait states, to another register, or when a
    later MFMA writes the register first, it is not."""
    mfma = "v_mfma_f32_16x16x32_bf16 v[4:7], v[8:11], v[12:15], 0"
    fill = ["v_mov_b32 v40, 0"] * 7
    assert len(mfma_result_hazards([mfma, "v_and_or_b32 v5, v1, v2, v3"])) == 1
    assert len(mfma_result_hazards([mfma] + fill + ["v_and_or_b32 v7, v1, v2, v3"])) == 1
    assert not mfma_result_hazards([mfma] + fill + ["v_mov_b32 v41, 0", "v_and_or_b32 v7, v1, v2, v3"])
    assert not mfma_result_hazards([mfma, "s_nop 7", "v_and_or_b32 v5, v1, v2, v3"])
    assert not mfma_result_hazards([mfma, "v_and_or_b32 v20, v1, v2, v3"])
    assert not mfma_result_hazards([mfma, "v_mfma_f32_16x16x32_bf16 v[4:7], v[8:11], v[12:15], 0",
                                    "s_nop 7", "v_and_or_b32 v5, v1, v2, v3"])


def test_kernel_sources_have_no_asm_instructions():
    """Every asm statement in the kernel sources is empty (it only makes a
    value opaque to the optimizer); no instruction is written in asm."""
    found = []
    for name in sorted(os.listdir(CSRC)):
        if not name.endswith((".hip", ".h")):
            continue
        with open(os.path.join(CSRC, name)) as f:
            for no, line in enumerate(f, 1):
                code = line.split("//")[0]
                for m in re.finditer(r"\basm\b\s*(?:volatile\s*)?\(\s*\"([^\"]*)\"", code):
                    if m.group(1).strip():
                        found.append("%s:%d: %s" % (name, no, line.strip()))
                if re.search(r"\basm\b", code) and not re.search(r"\basm\b\s*(?:volatile\s*)?\(\s*\"", code):
                    found.append("%s:%d: %s" % (name, no, line.strip()))
    assert not found, "asm with instructions: %s" % found


def test_built_library_has_no_valu_to_mfma_hazard():
    if not os.path.exists(LIB):
        pytest.skip("libqgemv.so is not built")
    for tool in ("llvm-objcopy", "llvm-objdump"):
        if not os.path.exists(os.path.join(LLVM, tool)):
            pytest.skip(tool + " not available")
    objs = _code_objects(LIB)
    assert objs, "no gfx950 code object in the library"
    mfmas, bad, overwritten = 0, [], []
    with tempfile.TemporaryDirectory() as d:
        for i, obj in enumerate(objs):
            path = os.path.join(d, "co%d.o" % i)
            with open(path, "wb") as f:
                f.write(obj)
            out = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", path],
                                 check=True, capture_output=True, text=True).stdout
            lines = _instruction_lines(out)
            mfmas += sum(1 for t in lines if t and t.startswith("v_mfma"))
            bad += mfma_hazards(lines)
            overwritten += mfma_result_hazards(lines)
    assert mfmas > 1000, "expected the MFMA kernels in the library (%d MFMAs found)" % mfmas
    assert not bad, "%d MFMAs read a VGPR written < %d wait states before, e.g. %s" % (
        len(bad), MIN_WAIT_STATES, bad[:3])
    assert not overwritten, "%d VALU writes land in an MFMA's result before it is written, e.g. %s" % (
        len(overwritten), overwritten[:3])
